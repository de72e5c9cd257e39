"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c calls every oracle entry point on small
inputs whose buffers have exactly the sizes the oracle's contract states,
with the defensive metadata cases (out-of-range and repeated LUT entries,
counts outside [0, max_kv], variable block sizes outside [0, block], empty
rows, shared metadata rows, zero and negative block scales, codebook-coded
K/V, unit subsets, rejected arguments).  It is built with gcc from the
oracle's own source and run as a separate process; any sanitizer finding
aborts it.  Host code only: nothing here touches a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")


def _sanitizers_available(tmp_path) -> bool:
    probe = tmp_path / "probe.c"
    probe.write_text("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", str(probe), "-o",
                        str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    if not _sanitizers_available(tmp_path):
        pytest.skip("gcc cannot link the address/undefined sanitizers here")
    exe = tmp_path / "oracle_sanitize"
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-Wall", "-Wextra", "-I", ORACLE_DIR, DRIVER,
         os.path.join(ORACLE_DIR, "bsa_oracle.c"), "-lm", "-o", str(exe)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # a preload of the surrounding environment would have to come before the
    # sanitizer runtime; the oracle run needs none
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env,
                         timeout=600)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report
    assert "runtime error" not in report, report
    assert "AddressSanitizer" not in report, report
    assert "all calls checked" in run.stdout
