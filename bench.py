"""Benchmark of the block-sparse attention forward on one MI355X.

A step is one forward pass over the video-shaped VSA workload: the launch
order pass (two small kernels: each head's units heaviest first) and the
forward kernel (decode, gather, QK^T, softmax, PV, epilogue).  Workload:
B=1, H=24, S=49152 (768 blocks of 64 tokens), D=128, bf16 N(0,1), 96 of 768
key blocks per query block (sorted LUT), variable_block_sizes uniform in
[16, 64].  Inputs are resident in HBM before the timed region starts.

Metric: effective TFLOP/s = 4*D*P / time, with P the exact number of
attended (query, key) pairs of the seeded metadata, against the MI355X bf16
dense MFMA peak (2.5 PFLOP/s): `value` over the whole step, the roofline's
`achieved` over the forward kernel alone (events around its launch).
Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--workload I] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_sparse_attention_tile_amd as bsa  # noqa: E402
import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
# the forward kernel and the launch-order pass (the order decides which
# units share the L2, so it changes the kernel's traffic)
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_attention_tile_amd", "csrc",
                               f) for f in ("bsa_fwd.hip", "bsa_device.h",
                                            "bsa_order.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bsa_fwd_traffic.json")


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the forward kernel's sources (the stored counter figures
    apply only to the kernel they were taken on)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def selected_matrix(w) -> torch.Tensor:
    """[n_units, NK] bool: key block kb is selected by unit u (set semantics:
    LUT entries below the clamped count, inside [0, NK))."""
    NQ, NK = w.NQ, w.NK
    u = torch.arange(w.n_units)
    qb, h, b = u % NQ, (u // NQ) % w.H, u // (NQ * w.H)
    if w.form == "lut":
        sb, sh = w.meta_strides
        rows = b * sb + h * sh + qb
        idx = w.q2k_idx.long()[rows]
        n = w.q2k_num.long()[rows].clamp(0, idx.shape[-1])
        ok = (torch.arange(idx.shape[-1])[None, :] < n[:, None]) & \
             (idx >= 0) & (idx < NK)
        sel = torch.zeros((w.n_units, NK + 1), dtype=torch.bool)
        sel.scatter_(1, torch.where(ok, idx, torch.full_like(idx, NK)),
                     torch.ones_like(ok))
        return sel[:, :NK]
    sb, sh = w.mask_strides
    rows = b * sb + h * sh + qb
    return w.mask[rows] != 0


def attended_pairs(w, units=None) -> int:
    """Exact number of attended (query, key) pairs (per unit: block query
    rows times the valid keys of its selected blocks)."""
    sel = selected_matrix(w)
    if units is not None:
        sel = sel[torch.as_tensor(units, dtype=torch.long)]
    nv = torch.full((w.NK,), w.block, dtype=torch.long) if w.vbs is None \
        else w.vbs.long().clamp(0, w.block)
    return int((sel.long() * nv[None, :]).sum()) * w.block


def _valid_counts(w) -> torch.Tensor:
    return torch.full((w.NK,), w.block, dtype=torch.long) if w.vbs is None \
        else w.vbs.long().clamp(0, w.block)


def issued_tile_flop(w) -> float:
    """Matrix-core work the forward kernel issues, counted in whole 32-key
    tiles (4*D*block*32 per tile): bf16 K/V tiles are cut from each unit's
    stream of valid keys, fp8 and scaled (codebook) K/V tiles from one block
    at a time."""
    sel = selected_matrix(w).long()
    nv = _valid_counts(w)
    if w.kv_fp8 or w.kv_codebook:
        tiles = int((sel * ((nv + 31) // 32)[None, :]).sum())
    else:
        tiles = int(((sel * nv[None, :]).sum(1) + 31).div(32, rounding_mode="floor").sum())
    return 4.0 * w.D * w.block * 32 * tiles


def compulsory_bytes(w) -> int:
    """Bytes every forward pass must move at least once: Q, O and the LSE,
    the valid K/V rows of every block some unit selects (with their scales),
    and the selection metadata."""
    sel = selected_matrix(w).view(w.B, w.Hk, (w.H // w.Hk) * w.NQ, w.NK).any(2)
    rows = int((sel.long() * _valid_counts(w)[None, None, :]).sum())
    row_bytes = w.k.shape[-1] * w.k.element_size()
    kv = 2 * rows * row_bytes
    if w.k_scale is not None:
        kv += 2 * int(sel.sum()) * 4
    q = w.q.numel() * w.q.element_size()
    meta = (w.q2k_idx.numel() * 4 + w.q2k_num.numel() * 4) if w.form == "lut" \
        else w.mask.numel()
    if w.vbs is not None:
        meta += w.vbs.numel() * 4
    return 2 * q + w.B * w.H * w.S * 4 + kv + meta


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def codebook_recode(w, kind: str):
    """The workload with its K/V re-coded as codebook codes (seeded
    bf16-exact codebooks of 256 (i8) or 16 (i4) levels, per-block scales)."""
    g = torch.Generator().manual_seed(1000)
    bits = 8 if kind == "i8cb" else 4
    kc = workloads.make_codebook(g, 1 << bits)
    vc = workloads.make_codebook(g, 1 << bits)
    src_k = w.k.float() * (w.k_scale.repeat_interleave(w.block, -1)[..., None]
                           if w.k_scale is not None else 1.0)
    src_v = w.v.float() * (w.v_scale.repeat_interleave(w.block, -1)[..., None]
                           if w.v_scale is not None else 1.0)
    w.k, w.k_scale = workloads.quantize_codebook_per_block(src_k, w.block, kc, bits)
    del src_k
    w.v, w.v_scale = workloads.quantize_codebook_per_block(src_v, w.block, vc, bits)
    w.k_codebook, w.v_codebook = kc, vc
    w.name = f"{w.name}_{kind}"
    return w


def launch(w, d, out, lse, kernel_events=None, fp8_route="auto"):
    """One forward pass; lse=None is the inference route (no LSE store).
    Codebook-coded K/V are dequantised inside the call.  The LUT form first
    computes its launch order on the GPU (heaviest units first, part of the
    step) when the launch has more units than run at once, in either form.
    kernel_events=(start, end): recorded around the forward call alone
    (after the order pass).  fp8_route: how fp8 K/V are widened (the
    binding's ``fp8_route``)."""
    cb = dict(k_codebook=d.get("k_codebook"), v_codebook=d.get("v_codebook"))
    order = None
    if bsa.api.launch_order_pays(w.B, w.H, w.NQ):
        if w.form == "lut":
            order = bsa.bsa_unit_order_lut(d["q2k_idx"], d["q2k_num"], d["vbs"],
                                           B=w.B, H=w.H, S=w.S, Sk=w.Sk,
                                           block=w.block,
                                           meta_strides=w.meta_strides)
        else:
            order = bsa.bsa_unit_order_bitmap(d["mask"], d["vbs"], B=w.B, H=w.H,
                                              S=w.S, Sk=w.Sk, block=w.block,
                                              mask_strides=w.mask_strides)
    if kernel_events is not None:
        kernel_events[0].record()
    if w.form == "lut":
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        d["vbs"], block=w.block, sm_scale=w.sm_scale,
                        k_scale=d["k_scale"], v_scale=d["v_scale"], **cb,
                        meta_strides=w.meta_strides, out=out, lse=lse,
                        need_lse=lse is not None, balance=False,
                        qblock_order=order, fp8_route=fp8_route)
    else:
        bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                           block=w.block, sm_scale=w.sm_scale,
                           k_scale=d["k_scale"], v_scale=d["v_scale"], **cb,
                           mask_strides=w.mask_strides, out=out, lse=lse,
                           need_lse=lse is not None, balance=False,
                           qblock_order=order, fp8_route=fp8_route)
    if kernel_events is not None:
        kernel_events[1].record()


def kv_route(w, args):
    """How the step turns the workload's K/V into the kernel's operands."""
    if args.kv or w.kv_codebook:
        return "codebook dequantisation pass, then the scaled-bf16 kernel"
    if w.kv_fp8:
        if bsa.api._widen_fp8(w.B, w.H, w.NQ, args.fp8_route):
            return "fp8 widening pass, then the scaled-bf16 kernel"
        return "fp8 widened inside the kernel"
    return "bf16"


def stored_counters(workload_name: str) -> dict:
    """The committed rocprofv3 counter record of the forward kernel on a
    workload, if it was taken on the current kernel source; else {}."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    e = t.get(workload_name)
    if not e or e.get("kernel_sha256_16") != kernel_hash():
        return {}
    return e


def stored_traffic(workload_name: str):
    """HBM bytes per launch from the committed counter record, or None."""
    return stored_counters(workload_name).get("hbm_bytes_per_launch")


def _counter_means(csv_path: str, counter: str, kernel_substr: str):
    """Mean of one rocprofv3 counter over the dispatches of a kernel."""
    import csv
    vals = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {csv_path}")
    return sum(vals) / len(vals), len(vals)


def record_traffic(pmc_dir: str, workload: int) -> int:
    """Turns four rocprofv3 --pmc runs under pmc_dir (copy_fetch, copy_write:
    this script's --copy-calibration; fetch, write: this script on the
    workload) into HBM bytes per launch of the forward kernel, each counter
    scaled by what it reads for a copy of exactly 1 GiB read + 1 GiB
    written, and stores them in the traffic file under the workload name,
    keyed to the current kernel source.  A fifth run under ``hit``
    (TCC_HIT_sum, TCC_MISS_sum), when present, adds the L2 hit rate."""
    csv_of = lambda n: os.path.join(pmc_dir, n, "run_counter_collection.csv")
    gib = float(1 << 30)
    cf, _ = _counter_means(csv_of("copy_fetch"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _counter_means(csv_of("copy_write"), "WRITE_SIZE", "copyBuffer")
    f_fac, w_fac = gib / (cf * 1024.0), gib / (cw * 1024.0)
    kf, nf = _counter_means(csv_of("fetch"), "FETCH_SIZE", "bsa_fwd_kernel")
    kw, nw = _counter_means(csv_of("write"), "WRITE_SIZE", "bsa_fwd_kernel")
    fetch = kf * 1024.0 * f_fac
    write = kw * 1024.0 * w_fac
    hit_rate = None
    if os.path.exists(csv_of("hit")):
        # optional fifth run: TCC_HIT_sum and TCC_MISS_sum on the workload
        hit, _ = _counter_means(csv_of("hit"), "TCC_HIT_sum", "bsa_fwd_kernel")
        miss, _ = _counter_means(csv_of("hit"), "TCC_MISS_sum", "bsa_fwd_kernel")
        hit_rate = round(hit / (hit + miss), 4) if hit + miss > 0 else None
    name = workloads.CONFIG_NAMES[workload]
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[name] = {
        "kernel_sha256_16": kernel_hash(),
        "hbm_bytes_per_launch": round(fetch + write),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "fetch_scale": round(f_fac, 4),
        "write_scale": round(w_fac, 4),
        "dispatches_averaged": [nf, nw],
    }
    if hit_rate is not None:
        table[name]["l2_hit_rate"] = hit_rate
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({name: table[name]}))
    return 0


def cpu_baseline(w, target_s: float):
    """The oracle (as it stands) on a bounded sample of the same workload's
    work units; throughput in the same unit as the GPU metric."""
    import numpy as np

    import oracle
    g = np.random.default_rng(1234)
    order = g.permutation(w.n_units)
    kw = dict(block=w.block, sm_scale=w.sm_scale, k_scale=w.k_scale,
              v_scale=w.v_scale, k_codebook=w.k_codebook,
              v_codebook=w.v_codebook)

    def run(units):
        t0 = time.perf_counter()
        if w.form == "lut":
            oracle.fwd_lut(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs,
                           meta_strides=w.meta_strides, units=units, **kw)
        else:
            oracle.fwd_bitmap(w.q, w.k, w.v, w.mask, w.vbs,
                              mask_strides=w.mask_strides, units=units, **kw)
        return time.perf_counter() - t0

    threads = oracle.num_threads()
    probe = order[:max(1, threads)].tolist()
    t_probe = run(probe)
    per_unit = t_probe / len(probe)
    n = int(min(w.n_units, max(len(probe), target_s / max(per_unit, 1e-6))))
    units = order[:n].tolist()
    progress(f"cpu baseline: oracle on {n} of {w.n_units} units "
             f"({threads} threads, ~{per_unit * n:.1f} s)")
    dt = run(units)
    pairs = attended_pairs(w, units)
    return {
        "value": 4.0 * w.D * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"{n} of {w.n_units} work units (b,h,q-block) of "
                   f"{w.name}, drawn at random (seed 1234); {pairs} attended "
                   f"pairs in {dt:.2f} s, fp64 C oracle with OpenMP"),
    }


def bench_mask_to_lut(args) -> int:
    """Times the block-map compaction on the selection matrix of a named
    workload (one row per work unit).  HBM-bound integer kernel: algorithmic
    bytes = mask read (1 B per entry) + LUT write (4 B per entry) + counts."""
    progress(f"generating workload {args.workload}")
    w = workloads.make_config(args.workload)
    mask = selected_matrix(w).to(torch.int8).cuda()
    rows, nk = mask.shape
    nbytes = rows * nk * 5 + rows * 4
    for _ in range(args.warmup):
        bsa.bsa_mask_to_lut(mask)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        bsa.bsa_mask_to_lut(mask)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "block-map -> LUT compaction, GB/s of mask read + LUT write",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8->i32",
        "data": "synthetic",
        "config": {"workload": f"mask_to_lut of {w.name} selection",
                   "rows": rows, "nk": nk, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }), flush=True)
    return 0


def bench_bwd(args) -> int:
    """Times the backward pass (delta pass, selection map, dq, dk/dv kernels)
    on a named bf16 workload, after one forward pass that supplies O and
    the LSE.  Algorithmic work: 5 products of 2*D flop per attended pair
    (S recompute, dP, dV, dK, dQ) = 10*D*P."""
    progress(f"generating workload {args.workload}")
    w = workloads.make_config(args.workload)
    if w.kv_fp8:
        print("the backward pass takes bf16 K/V", file=sys.stderr)
        return 2
    pairs = attended_pairs(w)
    flop = 10.0 * w.D * pairs
    dev = torch.device("cuda:0")
    d = {n: (None if getattr(w, n) is None else getattr(w, n).to(dev))
         for n in ("q", "k", "v", "q2k_idx", "q2k_num", "mask", "vbs")}
    d["k_scale"] = d["v_scale"] = None
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    launch(w, d, out, lse)
    g = torch.Generator().manual_seed(1)
    dout = torch.randn(tuple(w.q.shape), generator=g).to(torch.bfloat16).to(dev)
    kw = dict(block=w.block, variable_block_sizes=d["vbs"], sm_scale=w.sm_scale)
    if w.form == "lut":
        kw.update(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"],
                  meta_strides=w.meta_strides)
    else:
        kw.update(mask=d["mask"], meta_strides=w.mask_strides)
    need = int(bsa._lib.load().bsa_bwd_workspace_size(w.B, w.H, w.S, w.Sk,
                                                       w.block))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step():
        return bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse,
                           workspace=ws, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    tflops = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "effective TFLOP/s (10*D*attended pairs) + % bf16 MFMA peak, "
                  "VSA backward",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S,
                   "D": w.D, "block": w.block, "form": w.form,
                   "attended_pairs": pairs, "effective_flop_per_step": flop,
                   "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock ramps over the first launches: warm up well past it
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2,
                    help="named workload index (default 2: video-shaped VSA)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv", default=None, choices=("i8cb", "i4cb"),
                    help="re-code the workload's K/V as i8 / packed-i4 "
                         "codebook codes (each step then includes the "
                         "dequantisation pass)")
    ap.add_argument("--fp8-route", default="auto", choices=bsa.api.FP8_ROUTES,
                    help="fp8 K/V: widened inside the kernel, in a pass of "
                         "their own first, or by launch size (auto)")
    ap.add_argument("--no-lse", action="store_true",
                    help="inference route: the forward pass without the LSE "
                         "output")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--flush-cache", action="store_true",
                    help="forward only: overwrite 512 MB before every timed "
                         "launch and time each launch alone (cold L2 and MALL)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (the "
                         "reference kernel for scaling HBM byte counters)")
    ap.add_argument("--op", default="fwd",
                    choices=("fwd", "bwd", "mask_to_lut"),
                    help="fwd (default): the forward pass; bwd: the backward "
                         "pass; mask_to_lut: the block-map compaction on the "
                         "workload's selection")
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="no GPU work: read rocprofv3 FETCH_SIZE/WRITE_SIZE "
                         "runs from PMC_DIR and store the workload's HBM "
                         "bytes per launch")
    args = ap.parse_args()

    if args.record_traffic:
        return record_traffic(args.record_traffic, args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward pass runs on a "
              "single MI355X (each GPU would take its own share of heads "
              "with no communication); --gpus must be 1.",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.op == "mask_to_lut":
        return bench_mask_to_lut(args)
    if args.op == "bwd":
        return bench_bwd(args)
    if args.copy_calibration:
        n = 1 << 29  # 2**29 bf16 = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        progress("copy calibration: 3 copies of 1 GiB")
        return 0

    progress(f"generating workload {args.workload}")
    w = workloads.make_config(args.workload)
    if args.kv:
        progress(f"re-coding K/V as {args.kv}")
        w = codebook_recode(w, args.kv)
    pairs = attended_pairs(w)
    flop = 4.0 * w.D * pairs
    dev = torch.device("cuda:0")
    d = {n: (None if getattr(w, n) is None else getattr(w, n).to(dev))
         for n in ("q", "k", "v", "k_scale", "v_scale", "q2k_idx", "q2k_num",
                   "mask", "vbs", "k_codebook", "v_codebook")}
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device=dev)
    lse = None if args.no_lse else torch.empty((w.B, w.H, w.S),
                                               dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    progress(f"warmup {args.warmup} steps on {w.name}")
    for _ in range(args.warmup):
        launch(w, d, out, lse, fp8_route=args.fp8_route)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if args.flush_cache:
        # cold caches: a 512 MB write (twice the MALL) before every launch,
        # outside the timed interval of that launch
        scrub = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        pairs_ev = [(torch.cuda.Event(enable_timing=True),
                     torch.cuda.Event(enable_timing=True))
                    for _ in range(args.steps)]
        for i in range(args.steps):
            scrub.fill_(float(i))
            pairs_ev[i][0].record(stream)
            launch(w, d, out, lse, fp8_route=args.fp8_route)
            pairs_ev[i][1].record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in pairs_ev) / args.steps
        del scrub
        ms_kernel = None
        kernel_stats = None
    else:
        kev = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        ev0.record(stream)
        for i in range(args.steps):
            launch(w, d, out, lse, kernel_events=kev[i], fp8_route=args.fp8_route)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        # the forward kernel alone (the dominant kernel of the step)
        per_launch = sorted(a.elapsed_time(b) for a, b in kev)
        ms_kernel = sum(per_launch) / args.steps
        n = len(per_launch)
        kernel_stats = {
            "mean": round(ms_kernel, 5),
            "median": round((per_launch[(n - 1) // 2] + per_launch[n // 2]) / 2, 5),
            "min": round(per_launch[0], 5),
            "max": round(per_launch[-1], 5),
        }
    wall = time.perf_counter() - t0
    progress(f"timed {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)"
             + ("" if ms_kernel is None else
                f", forward kernel {ms_kernel:.4f} ms"))

    tflops = flop / (ms * 1e-3) / 1e12
    k_tflops = tflops if ms_kernel is None else flop / (ms_kernel * 1e-3) / 1e12
    counters = stored_counters(w.name)
    traffic = counters.get("hbm_bytes_per_launch")
    compulsory = compulsory_bytes(w)
    result = {
        "metric": "effective TFLOP/s (4*D*attended pairs) + % bf16 MFMA peak, "
                  "VSA fwd",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3-kv/bf16" if w.kv_fp8 else
                  f"{args.kv}-kv/bf16" if args.kv else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "H": w.H, "S": w.S, "D": w.D, "block": w.block,
            "form": w.form, "need_lse": not args.no_lse,
            "caches": "flushed before each launch" if args.flush_cache else "warm",
            "attended_pairs": pairs,
            "effective_flop_per_step": flop,
            "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
            "issued_tile_flop_per_step": issued_tile_flop(w),
            "compulsory_bytes": compulsory,
            "compulsory_gbs": round(compulsory / (ms * 1e-3) / 1e9, 1),
            "fabric_gbs": (None if traffic is None else
                           round(traffic / (ms * 1e-3) / 1e9, 1)),
            "l2_hit_rate": counters.get("l2_hit_rate"),
            "launch_order": ("heaviest units first (order pass in the step)"
                             if bsa.api.launch_order_pays(w.B, w.H, w.NQ)
                             else "q-block"),
            "key_split": (w.block == 64 and not (w.kv_fp8 or args.kv) and
                          w.n_units <= bsa.BSA_FWD_KEY_SPLIT_MAX_UNITS),
            "kv_route": kv_route(w, args),
            "fwd_kernel_ms": None if ms_kernel is None else round(ms_kernel, 5),
            # per-launch forward kernel times over the timed steps (HIP events
            # on the launch stream)
            "fwd_kernel_ms_stats": kernel_stats,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(k_tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
