"""Host-side logic of bench.py (CPU): the exact attended-pair count that the
effective-FLOP metric divides by agrees with the oracle's integer decode."""

import numpy as np
import pytest

import bench
import oracle
import workloads


def _oracle_pairs(w, units=None):
    kw = dict(B=w.B, H=w.H, S=w.S, block=w.block, vbs=w.vbs, units=units)
    if w.form == "lut":
        c = oracle.key_counts(q2k_idx=w.q2k_idx, q2k_num=w.q2k_num,
                              meta_strides=w.meta_strides, **kw)
    else:
        c = oracle.key_counts(mask=w.mask, mask_strides=w.mask_strides, **kw)
    return int(c.astype(np.int64).sum()) * w.block


@pytest.mark.parametrize("kw", [
    dict(seed=1, S=512, block=64, count_mode="uniform", vbs_mode="random"),
    dict(seed=2, S=512, block=128, form="bitmap", density=0.4,
         vbs_mode="zero_some"),
    dict(seed=3, S=512, block=64, shared_meta=True, density=0.5),
    dict(seed=4, S=512, block=64, max_kv=3, count_mode="uniform",
         pad_value=99),
])
def test_attended_pairs_matches_oracle_decode(kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), B=2, H=3, **kw)
    assert bench.attended_pairs(w) == _oracle_pairs(w)
    units = [0, 3, 7, w.n_units - 1]
    assert bench.attended_pairs(w, units) == _oracle_pairs(w, units)


def test_tiny_named_workload_pair_count_closed_form():
    w = workloads.make_config(0)
    # 8 q-blocks x 4 selected blocks; block 7 has 40 valid keys, others 64
    sel = bench.selected_matrix(w).numpy()
    want = sum(64 * (40 if kb == 7 else 64)
               for u in range(8) for kb in range(8) if sel[u, kb])
    assert bench.attended_pairs(w) == want == _oracle_pairs(w)


def test_tiny_named_workload_issued_tiles_and_compulsory_bytes():
    w = workloads.make_config(0)
    sel = bench.selected_matrix(w).numpy()
    # stream tiles: each unit's valid keys cut into 32-key tiles
    tiles = sum(-(-sum(40 if kb == 7 else 64 for kb in range(8) if sel[u, kb])
                  // 32) for u in range(8))
    assert bench.issued_tile_flop(w) == 4.0 * 128 * 64 * 32 * tiles
    # Q and O bf16, the LSE, the valid rows of every selected block of K and
    # V once (bf16 rows of 256 bytes), the LUT (8 x 8 int32), counts, vbs
    used = [kb for kb in range(8) if sel[:, kb].any()]
    kv_rows = sum(40 if kb == 7 else 64 for kb in used)
    want = 2 * 512 * 128 * 2 + 512 * 4 + 2 * kv_rows * 256 + 8 * 8 * 4 + 8 * 4 + 8 * 4
    assert bench.compulsory_bytes(w) == want


def test_fp8_tiles_are_per_block():
    w = workloads.make_random(5, B=1, H=2, S=512, block=64, kv="fp8",
                              vbs_mode="random", density=0.5)
    sel = bench.selected_matrix(w).numpy()
    nv = w.vbs.tolist()
    # one block per tile: a block with 1-32 valid keys is one tile, 33-64 two
    tiles = 0
    for u in range(w.n_units):
        for kb in range(w.NK):
            if sel[u, kb] and nv[kb] > 0:
                tiles += 1 if nv[kb] <= 32 else 2
    assert bench.issued_tile_flop(w) == 4.0 * 128 * 64 * 32 * tiles
    assert bench.issued_tile_flop(w) >= 4.0 * 128 * bench.attended_pairs(w)


def _counter_csv(path, rows):
    import os
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for kernel, counter, value in rows:
            f.write(f'"{kernel}","{counter}",{value}\n')


def test_record_traffic_scales_counters_by_the_copy_calibration(tmp_path,
                                                                monkeypatch):
    import json
    gib_kib = float(1 << 20)
    kern = "void bsa_fwd_kernel<64, 0, false>(FwdParams)"
    _counter_csv(tmp_path / "copy_fetch", [("__amd_rocclr_copyBuffer",
                                            "FETCH_SIZE", gib_kib / 2)])
    _counter_csv(tmp_path / "copy_write", [("__amd_rocclr_copyBuffer",
                                            "WRITE_SIZE", gib_kib)])
    _counter_csv(tmp_path / "fetch", [(kern, "FETCH_SIZE", 1000.0),
                                      (kern, "FETCH_SIZE", 3000.0)])
    _counter_csv(tmp_path / "write", [(kern, "WRITE_SIZE", 500.0)])
    _counter_csv(tmp_path / "hit", [(kern, "TCC_HIT_sum", 30.0),
                                    (kern, "TCC_MISS_sum", 70.0)])
    table = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    monkeypatch.setattr(bench, "kernel_hash", lambda: "feedfacefeedface")
    assert bench.record_traffic(str(tmp_path), 2) == 0
    e = json.load(open(table))[workloads.CONFIG_NAMES[2]]
    # the copy's FETCH_SIZE shows half of the GiB it read: fetch counts x2
    assert e["fetch_bytes_per_launch"] == 2 * 2000 * 1024
    assert e["write_bytes_per_launch"] == 500 * 1024
    assert e["hbm_bytes_per_launch"] == 2 * 2000 * 1024 + 500 * 1024
    assert e["dispatches_averaged"] == [2, 1]
    assert e["l2_hit_rate"] == 0.3
    assert bench.stored_traffic(workloads.CONFIG_NAMES[2]) == e["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0000000000000000")
    assert bench.stored_traffic(workloads.CONFIG_NAMES[2]) is None  # stale source


def test_multi_gpu_request_exits_with_message(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
