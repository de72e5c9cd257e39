"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element.  Tolerances: O max-abs 1e-2, LSE
(base 2) 1e-3 absolute; rows with no attended key bit-exact (+0 and the
sentinel).  Outputs are pre-filled with NaN so unwritten elements fail."""

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from tests.gpu_helpers import (check, gather_units, log, run_gpu, run_oracle,
                               scaled_input_bounds, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL = [
    # (label, make_random kwargs)
    ("lut64_half", dict(seed=101, B=1, H=2, S=512, block=64, density=0.5)),
    ("lut64_full_dense", dict(seed=102, B=2, H=1, S=256, block=64, density=1.0)),
    ("lut64_vbs_random", dict(seed=103, B=1, H=3, S=768, block=64,
                              count_mode="uniform", vbs_mode="random")),
    ("lut64_vbs_zero_some", dict(seed=104, B=2, H=2, S=512, block=64,
                                 count_mode="uniform", vbs_mode="zero_some")),
    ("lut128_uniform", dict(seed=105, B=1, H=2, S=1024, block=128,
                            count_mode="uniform", vbs_mode="partial")),
    ("lut128_dense", dict(seed=106, B=1, H=1, S=512, block=128, density=1.0)),
    ("lut64_maxkv1", dict(seed=107, B=1, H=2, S=512, block=64, max_kv=1,
                          count_mode="uniform")),
    ("lut64_shared_meta", dict(seed=108, B=2, H=3, S=512, block=64,
                               shared_meta=True, density=0.4,
                               vbs_mode="partial")),
    ("lut64_count_zero", dict(seed=109, B=1, H=2, S=256, block=64,
                              count_mode="zero")),
    ("lut64_one_block", dict(seed=110, B=1, H=2, S=64, block=64, density=1.0,
                             vbs_mode="partial")),
    ("lut64_std3", dict(seed=111, B=1, H=2, S=512, block=64, density=0.5,
                        std=3.0, vbs_mode="partial")),
    ("bitmap64", dict(seed=112, B=1, H=2, S=512, block=64, form="bitmap",
                      density=0.5, vbs_mode="random")),
    ("bitmap128_shared", dict(seed=113, B=2, H=2, S=1024, block=128,
                              form="bitmap", shared_meta=True, density=0.3)),
    ("fp8_lut64", dict(seed=114, B=1, H=2, S=512, block=64, kv="fp8",
                       density=0.5, vbs_mode="partial")),
    ("fp8_lut128", dict(seed=115, B=2, H=1, S=512, block=128, kv="fp8",
                        count_mode="uniform", vbs_mode="random")),
    ("fp8_bitmap64", dict(seed=116, B=1, H=2, S=512, block=64, kv="fp8",
                          form="bitmap", density=0.6)),
    ("lut64_long_nk1024", dict(seed=117, B=1, H=1, S=65536, block=64,
                               max_kv=40, density=0.0006, count_mode="uniform",
                               vbs_mode="partial")),
    # grouped K/V heads (query head h reads K/V head h // (H // Hk)) and
    # query length != key length
    ("gqa_lut64", dict(seed=118, B=2, H=4, Hk=2, S=512, block=64,
                       count_mode="uniform", vbs_mode="random")),
    ("gqa_bitmap128", dict(seed=119, B=1, H=6, Hk=1, S=1024, block=128,
                           form="bitmap", density=0.4, vbs_mode="partial")),
    ("rect_q_short", dict(seed=120, B=1, H=2, S=256, Sk=1024, block=64,
                          density=0.5, vbs_mode="partial")),
    ("rect_q_long", dict(seed=121, B=2, H=2, Hk=1, S=1024, Sk=256, block=64,
                         count_mode="uniform", vbs_mode="zero_some")),
    ("gqa_fp8_rect", dict(seed=122, B=1, H=4, Hk=2, S=512, Sk=768, block=64,
                          kv="fp8", density=0.5, vbs_mode="random")),
    ("gqa_rect128_shared", dict(seed=123, B=2, H=4, Hk=4, S=512, Sk=1536,
                                block=128, shared_meta=True, density=0.3)),
    # valid counts around tile and half-tile edges, and runs of very short
    # blocks: 32-row tiles of the key stream span many blocks
    ("lut64_vbs_edges", dict(seed=124, B=1, H=2, S=2048, block=64,
                             density=0.6, vbs_mode="edges")),
    ("lut64_vbs_tiny", dict(seed=125, B=1, H=2, S=4096, block=64,
                            density=0.9, vbs_mode="tiny")),
    ("lut128_vbs_edges", dict(seed=126, B=1, H=2, S=2048, block=128,
                              count_mode="uniform", vbs_mode="edges")),
    ("bitmap128_vbs_tiny", dict(seed=127, B=1, H=2, S=4096, block=128,
                                form="bitmap", density=0.7, vbs_mode="tiny")),
    ("gqa_rect64_vbs_edges", dict(seed=128, B=2, H=4, Hk=2, S=512, Sk=2048,
                                  block=64, density=0.5, vbs_mode="edges")),
    # ~230 selected blocks of 1-4 keys: tiles span many blocks and cross
    # the 64-entry list chunks in the middle of a tile
    ("lut64_many_tiny", dict(seed=129, B=1, H=1, S=1024, Sk=16384, block=64,
                             density=0.9, vbs_mode="tiny")),
    # lists of exactly 64, 65, 128 and 129 selected blocks of 1-4 keys: the
    # walk's list chunk and the one read ahead end exactly at, or one entry
    # past, a 64-entry boundary (key-split launches, then one with more
    # units than a split launch takes)
    ("lut64_list64", dict(seed=130, B=1, H=1, S=256, Sk=4096, block=64,
                          density=1.0, vbs_mode="tiny")),
    ("lut64_list65", dict(seed=131, B=1, H=2, S=256, Sk=4160, block=64,
                          density=1.0, vbs_mode="tiny")),
    ("bitmap64_list128", dict(seed=132, B=1, H=1, S=512, Sk=8192, block=64,
                              form="bitmap", density=1.0, vbs_mode="tiny")),
    ("lut64_list129", dict(seed=133, B=1, H=1, S=512, Sk=8256, block=64,
                           density=1.0, vbs_mode="tiny")),
    ("wide_lut64_list129", dict(seed=134, B=1, H=9, S=4096, Sk=8256, block=64,
                                density=1.0, vbs_mode="tiny")),
]


@pytest.mark.parametrize("label,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_random_parity(label, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    log(f"[parity] {label} B{w.B} H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk} blk{w.block} form={w.form} "
        f"fp8={w.kv_fp8}")
    out, lse = run_gpu(w)
    units = None
    if w.n_units > 64:
        units = sorted(set(np.linspace(0, w.n_units - 1, 48).astype(int).tolist()))
    o_ref, l_ref = run_oracle(w, units=units)
    if units is None:
        o_gpu = out.float().cpu().numpy()
        l_gpu = lse.cpu().numpy()
    else:
        o_gpu, l_gpu = gather_units(w, out, lse, units)
    if kw.get("std", 1.0) > 1.0:
        # inputs scaled beyond N(0, 1): bound derived from the bf16 roundings
        o_abs, o_rel = scaled_input_bounds(float(w.v.float().abs().max()))
        check(o_gpu, l_gpu, o_ref, l_ref, label, o_rel=o_rel, o_abs=o_abs)
    else:
        check(o_gpu, l_gpu, o_ref, l_ref, label)


# Launches on either side of BSA_FWD_KEY_SPLIT_MAX_UNITS at block 64 with
# bf16 K/V: "wide" ones (more units) run one wave group per unit, "split"
# ones divide every unit's selected blocks between two wave groups and merge
# the partial results.  Each list holds ragged, empty and one-block rows.
KEY_SPLIT = [
    ("wide_lut64_vbs_edges", True, dict(seed=140, B=2, H=40, S=512, block=64,
                                         count_mode="uniform", vbs_mode="edges")),
    ("wide_bitmap64_vbs_tiny", True, dict(seed=141, B=1, H=72, S=512, block=64,
                                           form="bitmap", density=0.8,
                                           vbs_mode="tiny")),
    ("wide_gqa_lut64_zero_some", True, dict(seed=142, B=2, H=48, Hk=8, S=384,
                                             block=64, count_mode="uniform",
                                             vbs_mode="zero_some")),
    ("split_lut64_vbs_edges", False, dict(seed=143, B=2, H=4, S=1024, block=64,
                                           count_mode="uniform", vbs_mode="edges")),
    ("split_bitmap64_rect", False, dict(seed=144, B=1, H=4, Hk=2, S=1024,
                                         Sk=4096, block=64, form="bitmap",
                                         density=0.3, vbs_mode="partial")),
    # a few full blocks among many 1..4-key ones: the halves are cut at a
    # block boundary, far from half the blocks
    ("split_lut64_heavy_blocks", False, dict(seed=145, B=1, H=8, S=2048,
                                              block=64, density=0.7,
                                              vbs_mode="tiny")),
]


@pytest.mark.parametrize("label,wide,kw", KEY_SPLIT, ids=[c[0] for c in KEY_SPLIT])
def test_key_split_launch_parity(label, wide, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    if label.endswith("heavy_blocks"):
        w.vbs[::7] = 64
    assert (w.n_units > bsa.BSA_FWD_KEY_SPLIT_MAX_UNITS) == wide
    log(f"[parity] {label} units={w.n_units} B{w.B} H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk} "
        f"form={w.form}")
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    check(out.float().cpu().numpy(), lse.cpu().numpy(),
          o_ref.reshape(tuple(out.shape)), l_ref.reshape(tuple(lse.shape)), label)


# BSA_MAX_KEY_BLOCKS key blocks: the LDS byte map and block list at their
# largest, the list walked in 64-entry chunks to its end and per-lane load
# offsets up to the last block (512 MB into the K/V plane at block 128).
# Every row selects the first and the last block, both fully valid.
MAX_NK = [
    ("lut64_max_key_blocks", dict(seed=130, B=1, H=1, S=128, Sk=64 * 16384,
                                  block=64, density=300 / 16384,
                                  vbs_mode="partial")),
    ("bitmap128_max_key_blocks", dict(seed=131, B=1, H=2, Hk=1, S=256,
                                      Sk=128 * 16384, block=128, form="bitmap",
                                      density=0.01, vbs_mode="edges")),
]


@pytest.mark.parametrize("label,kw", MAX_NK, ids=[c[0] for c in MAX_NK])
def test_max_key_blocks_parity(label, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    assert w.NK == bsa.BSA_MAX_KEY_BLOCKS
    w.vbs[0] = w.vbs[-1] = w.block
    if w.form == "lut":
        w.q2k_idx[:, 0] = w.NK - 1
        w.q2k_idx[:, 1] = 0
    else:
        w.mask[:, 0] = 1
        w.mask[:, -1] = 1
    log(f"[parity] {label} H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk} blk{w.block} form={w.form}")
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, label)


def test_tiny_named_workload_full_parity():
    w = workloads.make_config(0)
    log(f"[parity] {w.name} (every element)")
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, w.name)


_FULL_SIZE = {}


def _full_size_gpu(cfg):
    """The named workload and its GPU outputs, launched exactly as the
    benchmark launches them (computed once per module)."""
    if cfg not in _FULL_SIZE:
        _FULL_SIZE.clear()
        w = workloads.make_config(cfg)
        log(f"[parity] {w.name}: B{w.B} H{w.H} S{w.S} blk{w.block} "
            f"units={w.n_units}")
        out, lse = run_gpu(w)
        # whole-output properties that hold at any size
        assert not torch.isnan(out).any().item(), "unwritten or NaN output"
        assert not torch.isnan(lse).any().item(), "unwritten or NaN lse"
        assert torch.isfinite(lse).all().item()
        _FULL_SIZE[cfg] = (w, out, lse)
    return _FULL_SIZE[cfg]


def _compare_units(w, out, lse, units, label):
    o_ref, l_ref = run_oracle(w, units=units)
    o_gpu, l_gpu = gather_units(w, out, lse, units)
    check(o_gpu, l_gpu, o_ref, l_ref, label)


# (config, chunk, chunks): every workload element by element, in chunks of
# work units (each chunk a few seconds of the oracle on the host's cores)
FULL_SIZE = ([(1, 0, 1)] + [(4, k, 4) for k in range(4)] +
             [(2, k, 8) for k in range(8)] + [(3, k, 4) for k in range(4)])


@pytest.mark.parametrize("cfg,chunk,chunks", FULL_SIZE,
                         ids=[f"cfg{c}" + ("" if k is None else f"_part{k}of{n}")
                              for c, k, n in FULL_SIZE])
def test_named_workload_parity(cfg, chunk, chunks):
    """Full-size named workloads, launched exactly as the benchmark launches
    them, compared with the oracle on every element: Jenga (1 024 units),
    fp8 (6 144), video (18 432, in eight chunks) and block 128 (10 240, in
    four), the heaviest, the lightest and the empty units among them."""
    w, out, lse = _full_size_gpu(cfg)
    per = (w.n_units + chunks - 1) // chunks
    units = list(range(chunk * per, min(w.n_units, (chunk + 1) * per)))
    log(f"  oracle on units {units[0]}..{units[-1]} of {w.n_units}")
    _compare_units(w, out, lse, units, f"{w.name}[{len(units)} units]")



def test_need_lse_false_gives_same_output_and_leaves_lse_alone():
    w = workloads.make_random(201, B=1, H=2, S=512, block=64,
                              count_mode="uniform", vbs_mode="partial")
    log("[parity] need_lse=False")
    out1, _ = run_gpu(w)
    out2, _ = run_gpu(w, need_lse=False)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_gpu_result_is_bitwise_invariant_to_lut_order_padding_duplicates():
    w = workloads.make_random(202, B=1, H=2, S=1024, block=64, max_kv=10,
                              count_mode="uniform", vbs_mode="random")
    log("[parity] LUT order / padding / duplicate invariance")
    out1, lse1 = run_gpu(w)
    idx = w.q2k_idx.clone()
    num = w.q2k_num.clone()
    g = torch.Generator().manual_seed(3)
    wide = torch.full((idx.shape[0], idx.shape[1] + 2), -7, dtype=torch.int32)
    for r in range(idx.shape[0]):
        n = int(num[r])
        row = idx[r, :n][torch.randperm(n, generator=g)]
        extra = [int(row[0])] if n > 0 else []
        extra.append(w.NQ + 11)  # out of range below the count: skipped
        full = torch.cat([row, torch.tensor(extra, dtype=torch.int32)])
        wide[r, :len(full)] = full
        garbage = [2**31 - 1, -2**31, 5, w.NQ, -1]
        npad = wide.shape[1] - len(full)
        wide[r, len(full):] = torch.tensor(
            [garbage[i % len(garbage)] for i in range(npad)], dtype=torch.int32)
        num[r] = len(full)
    w.q2k_idx, w.q2k_num = wide.contiguous(), num
    out2, lse2 = run_gpu(w)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_bitmap_form_is_bitwise_equal_to_compacted_lut():
    w = workloads.make_random(203, B=2, H=2, S=1024, block=64, form="bitmap",
                              density=0.35, vbs_mode="random")
    log("[parity] bitmap == compacted LUT")
    out1, lse1 = run_gpu(w)
    m = w.mask.numpy()
    idx = np.full(m.shape, -1, dtype=np.int32)
    num = np.zeros(m.shape[0], dtype=np.int32)
    for r in range(m.shape[0]):
        nz = np.nonzero(m[r])[0]
        idx[r, :len(nz)] = nz
        num[r] = len(nz)
    w.form = "lut"
    w.q2k_idx = torch.from_numpy(idx)
    w.q2k_num = torch.from_numpy(num)
    w.meta_strides = w.mask_strides
    out2, lse2 = run_gpu(w)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_out_of_range_counts_and_vbs_are_clamped_like_the_oracle():
    w = workloads.make_random(204, B=1, H=2, S=512, block=64, max_kv=5,
                              count_mode="uniform")
    num = w.q2k_num.clone()
    num[::3] = 1000   # above max_kv: clamped
    num[1::5] = -4    # negative: empty row
    w.q2k_num = num
    w.vbs = torch.tensor([64, 1000, -5, 65, 3, 0, 64, 200], dtype=torch.int32)
    log("[parity] clamped counts and vbs")
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
          "clamped")


def test_invalid_static_arguments_raise_and_write_nothing():
    w = workloads.make_random(205, B=1, H=1, S=256, block=64)
    d = to_dev(w)
    out = torch.full(tuple(w.q.shape), 7.0, dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((1, 1, 256), 7.0, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        block=32, out=out, lse=lse)
    assert e.value.status == bsa.BSA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all().item() and (lse == 7.0).all().item()


def test_binding_rejects_misplaced_or_short_buffers_before_launch():
    """The C ABI sees raw pointers only; the binding checks devices and
    sizes against what the kernels would read or write."""
    w = workloads.make_random(206, B=1, H=2, S=256, block=64,
                              vbs_mode="partial")
    d = to_dev(w)
    args = (d["q"], d["k"], d["v"])
    log("[binding] misplaced and short buffers")
    bad = [
        dict(q2k_idx=w.q2k_idx),                       # metadata on the host
        dict(q2k_idx=d["q2k_idx"][:3]),                # fewer rows than units
        dict(q2k_num=d["q2k_num"][:3]),
        dict(vbs=d["vbs"][:2]),                        # fewer than NK entries
        dict(out=torch.empty((1, 2, 128, 128), dtype=torch.bfloat16,
                             device="cuda")),          # wrong output shape
        dict(lse=torch.empty((1, 2, 256), dtype=torch.float16,
                             device="cuda")),          # wrong LSE dtype
    ]
    for over in bad:
        kw = dict(q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"], vbs=d["vbs"],
                  out=None, lse=None)
        kw.update(over)
        with pytest.raises(ValueError):
            bsa.bsa_fwd_lut(*args, kw["q2k_idx"], kw["q2k_num"], kw["vbs"],
                            block=64, out=kw["out"], lse=kw["lse"])
    mask = torch.ones((2 * 4, 3), dtype=torch.int8, device="cuda")  # NK is 4
    with pytest.raises(ValueError):
        bsa.bsa_fwd_bitmap(*args, mask, block=64)
    out, lse = bsa.bsa_fwd_lut(*args, d["q2k_idx"], d["q2k_num"], d["vbs"],
                               block=64)
    with pytest.raises(ValueError):
        bsa.bsa_bwd(*args, out, out[:, :1].contiguous(), lse, block=64,
                    q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"])
    torch.cuda.synchronize()

