"""GPU tests of the launch order of the work units (bsa_unit_order_lut,
bsa_unit_order_bitmap) and of the ordered forward entry points: the order is
exactly the host's stable sort of the attended-key counts, and the forward
outputs are bit-identical with and without it (each unit computes the same
bits in any order)."""

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from tests.gpu_helpers import log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def expected_order(w) -> np.ndarray:
    """Host reference of the order: per (b, h), q-blocks by decreasing rank
    value min(count // 64, 2^21 - 1) * 1024 + 1023 - mean (count = sum of
    the valid keys of the row's first clamp(num) in-range entries, repeats
    counted; mean = their block indices' sum * 1023 // (entries *
    max(NK - 1, 1))), ties by increasing q-block."""
    NQ, NK, B, H = w.NQ, w.NK, w.B, w.H
    idx = w.q2k_idx.numpy().reshape(-1, w.q2k_idx.shape[-1])
    num = w.q2k_num.numpy().reshape(-1)
    max_kv = idx.shape[1]
    vbs = (np.full(NK, w.block) if w.vbs is None
           else np.clip(w.vbs.numpy(), 0, w.block))
    sb, sh = w.meta_strides
    out = np.empty(B * H * NQ, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            work = []
            for qb in range(NQ):
                row = b * sb + h * sh + qb
                n = int(np.clip(num[row], 0, max_kv))
                e = idx[row, :n]
                e = e[(e >= 0) & (e < NK)]
                count = int(vbs[e].sum())
                mean = (int(e.astype(np.int64).sum()) * 1023 //
                        (len(e) * max(NK - 1, 1))) if len(e) else 0
                work.append(min(count // 64, 2**21 - 1) * 1024 + 1023 - mean)
            o = sorted(range(NQ), key=lambda i: (-work[i], i))
            out[(b * H + h) * NQ:(b * H + h + 1) * NQ] = o
    return out


def expected_order_bitmap(w) -> np.ndarray:
    """Host reference of the bitmap-form order: as expected_order, over the
    key blocks the unit's mask row selects (each once)."""
    NQ, NK, B, H = w.NQ, w.NK, w.B, w.H
    mask = w.mask.numpy().reshape(-1, NK)
    vbs = (np.full(NK, w.block) if w.vbs is None
           else np.clip(w.vbs.numpy(), 0, w.block))
    sb, sh = w.mask_strides
    out = np.empty(B * H * NQ, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            work = []
            for qb in range(NQ):
                e = np.nonzero(mask[b * sb + h * sh + qb])[0]
                count = int(vbs[e].sum())
                mean = (int(e.sum()) * 1023 // (len(e) * max(NK - 1, 1))
                        if len(e) else 0)
                work.append(min(count // 64, 2**21 - 1) * 1024 + 1023 - mean)
            o = sorted(range(NQ), key=lambda i: (-work[i], i))
            out[(b * H + h) * NQ:(b * H + h + 1) * NQ] = o
    return out


def gpu_order_bitmap(w, d):
    o = bsa.bsa_unit_order_bitmap(d["mask"], d["vbs"], B=w.B, H=w.H, S=w.S,
                                  Sk=w.Sk, block=w.block,
                                  mask_strides=w.mask_strides)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def gpu_order(w, d):
    o = bsa.bsa_unit_order_lut(d["q2k_idx"], d["q2k_num"], d["vbs"], B=w.B,
                               H=w.H, S=w.S, Sk=w.Sk, block=w.block,
                               meta_strides=w.meta_strides)
    torch.cuda.synchronize()
    return o.cpu().numpy()


CASES = [
    ("rand_lut64", dict(seed=301, B=2, H=3, S=64 * 37, block=64,
                        count_mode="uniform", vbs_mode="random")),
    ("rand_lut128_shared", dict(seed=302, B=2, H=2, S=128 * 20, block=128,
                                shared_meta=True, count_mode="uniform",
                                vbs_mode="partial")),
    ("rand_lut64_garbage", dict(seed=303, B=1, H=2, S=64 * 9, block=64,
                                count_mode="uniform", pad_value=2**31 - 1)),
    ("rand_lut64_one_qblock", dict(seed=304, B=2, H=2, S=64, block=64,
                                   count_mode="uniform")),
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_order_matches_host_sort(label, kw):
    w = workloads.make_random(**kw)
    if label == "rand_lut64_garbage":
        # below the count: entries out of range (skipped) and repeats
        # (counted twice by the estimate)
        idx, num = w.q2k_idx, w.q2k_num
        for r in range(idx.shape[0]):
            if num[r] >= 3 and r % 3 == 0:
                idx[r, 0] = w.NK + 3
                idx[r, 1] = -5
            elif num[r] >= 3 and r % 3 == 1:
                idx[r, 2] = idx[r, 1]
    log(f"[order] {label}: B={w.B} H={w.H} S={w.S} block={w.block}")
    d = to_dev(w)
    assert np.array_equal(gpu_order(w, d), expected_order(w))


@pytest.mark.parametrize("cfg", [2, 3])
def test_order_matches_host_sort_full_configs(cfg):
    w = workloads.make_config(cfg)
    log(f"[order] {w.name}")
    d = to_dev(w)
    assert np.array_equal(gpu_order(w, d), expected_order(w))


def test_order_at_the_query_block_limit():
    S = 64 * bsa.BSA_MAX_ORDER_QBLOCKS
    w = workloads.make_random(seed=305, B=1, H=1, S=S, block=64, max_kv=4,
                              count_mode="uniform", vbs_mode="random")
    log(f"[order] NQ = {w.NQ}")
    d = to_dev(w)
    assert np.array_equal(gpu_order(w, d), expected_order(w))


FWD_CASES = [
    ("rand_lut64", dict(seed=311, B=2, H=3, S=64 * 37, block=64,
                        count_mode="uniform", vbs_mode="random")),
    ("rand_lut128", dict(seed=312, B=1, H=3, S=128 * 21, block=128,
                         count_mode="uniform", vbs_mode="partial")),
    ("rand_lut64_shared_gqa", dict(seed=313, B=2, H=4, Hk=2, S=64 * 12,
                                   block=64, shared_meta=True,
                                   count_mode="uniform")),
]


@pytest.mark.parametrize("label,kw", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_ordered_forward_is_bitwise_the_unordered_one(label, kw):
    w = workloads.make_random(**kw)
    log(f"[order-fwd] {label}")
    d = to_dev(w)
    order = bsa.bsa_unit_order_lut(d["q2k_idx"], d["q2k_num"], d["vbs"],
                                   B=w.B, H=w.H, S=w.S, Sk=w.Sk, block=w.block,
                                   meta_strides=w.meta_strides)
    ident = torch.arange(w.NQ, dtype=torch.int32, device="cuda").repeat(w.B * w.H)
    assert not torch.equal(order, ident)  # the ordered launch differs
    outs = []
    for qo in (None, order):
        out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full((w.B, w.H, w.S), float("nan"), dtype=torch.float32,
                         device="cuda")
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        d["vbs"], block=w.block, sm_scale=w.sm_scale,
                        meta_strides=w.meta_strides, out=out, lse=lse,
                        balance=False, qblock_order=qo)
        torch.cuda.synchronize()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("cfg", [2, 3])
def test_ordered_forward_full_configs(cfg):
    w = workloads.make_config(cfg)
    log(f"[order-fwd] {w.name}")
    d = to_dev(w)
    assert bsa.api.launch_order_pays(w.B, w.H, w.NQ)
    a = run_gpu(w, dev_inputs=d)  # the binding orders by default
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
    bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                    d["vbs"], block=w.block, sm_scale=w.sm_scale,
                    meta_strides=w.meta_strides, out=out, lse=lse,
                    balance=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], out) and torch.equal(a[1], lse)


def test_out_of_range_order_entries_are_clamped():
    """Entries past NQ clamp to the last query block: every unit then
    computes that block (the same bits), which must match the reference."""
    w = workloads.make_random(seed=321, B=1, H=2, S=64 * 6, block=64,
                              count_mode="uniform", vbs_mode="random")
    d = to_dev(w)
    ref, ref_lse = run_gpu(w, dev_inputs=d)
    order = torch.full((w.B * w.H * w.NQ,), w.NQ + 7, dtype=torch.int32,
                       device="cuda")
    out = torch.zeros(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
    from block_sparse_attention_tile_amd import _lib
    from block_sparse_attention_tile_amd.api import _cur_stream, _ptr
    idx = d["q2k_idx"].to(torch.int32).contiguous()
    num = d["q2k_num"].to(torch.int32).contiguous()
    vbs = d["vbs"].to(torch.int32).contiguous()
    sb, sh = w.meta_strides
    rc = _lib.load().bsa_fwd_lut_ordered(
        _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]), 0, None, None, _ptr(idx),
        _ptr(num), int(idx.shape[-1]), int(sb), int(sh), _ptr(vbs),
        _ptr(order), float(w.sm_scale), _ptr(out), _ptr(lse), w.B, w.H, w.H,
        w.S, w.S, 128, w.block, _cur_stream(d["q"]))
    assert rc == bsa.BSA_OK
    torch.cuda.synchronize()
    last = slice((w.NQ - 1) * w.block, w.NQ * w.block)
    assert torch.equal(out[:, :, last], ref[:, :, last])
    assert torch.equal(lse[:, :, last], ref_lse[:, :, last])


def test_ordered_backward_is_bitwise_the_unordered_bitmap_form():
    """The LUT-form backward launches its dq units heaviest first; the
    bitmap form on the same selection keeps the q-block order.  Same set,
    same per-unit arithmetic: the gradients must agree bit for bit."""
    # more units (1 536) than run at once, so both kinds of backward unit
    # (query blocks and key blocks) are reordered
    w = workloads.make_random(331, B=1, H=24, S=64 * 64, block=64,
                              form="bitmap", density=0.5, vbs_mode="random")
    log("[order-bwd] LUT vs bitmap")
    mask = w.mask
    idx = torch.full((mask.shape[0], w.NK), -1, dtype=torch.int32)
    num = torch.zeros(mask.shape[0], dtype=torch.int32)
    for r in range(mask.shape[0]):
        sel = torch.nonzero(mask[r] != 0).flatten().to(torch.int32)
        idx[r, :len(sel)] = sel
        num[r] = len(sel)
    assert len(set(num.tolist())) > 1  # the order is not the identity
    d = to_dev(w)
    out, lse = run_gpu(w, dev_inputs=d)
    g = torch.Generator().manual_seed(12)
    dout = torch.randn(tuple(w.q.shape), generator=g).to(torch.bfloat16).cuda()
    common = dict(block=w.block, variable_block_sizes=d["vbs"],
                  sm_scale=w.sm_scale, meta_strides=w.mask_strides)
    g_bm = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse,
                       mask=d["mask"], **common)
    g_lut = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse,
                        q2k_idx=idx.cuda(), q2k_num=num.cuda(), **common)
    torch.cuda.synchronize()
    for a, b in zip(g_bm, g_lut):
        assert torch.equal(a, b)


LARGE = [
    # more units than run at once, so the binding orders them by default
    ("lut64_gqa", dict(seed=341, B=2, H=8, Hk=2, S=64 * 80, block=64,
                       count_mode="uniform", vbs_mode="random", max_kv=24)),
    ("lut128_shared", dict(seed=342, B=3, H=8, S=128 * 48, block=128,
                           shared_meta=True, count_mode="uniform",
                           vbs_mode="partial", max_kv=16)),
    ("lut64_rect_tiny", dict(seed=343, B=1, H=16, S=64 * 72, Sk=64 * 40,
                             block=64, count_mode="uniform", vbs_mode="tiny")),
    ("lut64_fp8", dict(seed=344, B=2, H=8, S=64 * 72, block=64, kv="fp8",
                       count_mode="uniform", max_kv=20)),
]


@pytest.mark.parametrize("label,kw", LARGE, ids=[c[0] for c in LARGE])
def test_default_ordered_launch_is_bitwise_the_qblock_order(label, kw):
    w = workloads.make_random(**kw)
    assert bsa.api.launch_order_pays(w.B, w.H, w.NQ)
    log(f"[order-large] {label}: units {w.n_units}")
    d = to_dev(w)
    res = []
    for balance in (True, False):
        out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full((w.B, w.H, w.S), float("nan"), dtype=torch.float32,
                         device="cuda")
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        d["vbs"], block=w.block, sm_scale=w.sm_scale,
                        k_scale=d["k_scale"], v_scale=d["v_scale"],
                        meta_strides=w.meta_strides, out=out, lse=lse,
                        balance=balance)
        torch.cuda.synchronize()
        res.append((out, lse))
    assert not torch.isnan(res[0][0].float()).any()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


BITMAP_CASES = [
    ("rand_bitmap64", dict(seed=321, B=2, H=3, S=64 * 37, block=64,
                           form="bitmap", density=0.4, vbs_mode="random")),
    ("rand_bitmap128_shared", dict(seed=322, B=2, H=2, S=128 * 20, block=128,
                                   form="bitmap", shared_meta=True,
                                   density=0.6, vbs_mode="partial")),
    ("rand_bitmap64_rect", dict(seed=323, B=1, H=2, S=64 * 9, Sk=64 * 70,
                                block=64, form="bitmap", density=0.1)),
]


@pytest.mark.parametrize("label,kw", BITMAP_CASES, ids=[c[0] for c in BITMAP_CASES])
def test_bitmap_order_matches_host_sort(label, kw):
    w = workloads.make_random(**kw)
    log(f"[order] {label}: B={w.B} H={w.H} S={w.S} Sk={w.Sk} block={w.block}")
    d = to_dev(w)
    assert np.array_equal(gpu_order_bitmap(w, d), expected_order_bitmap(w))


def test_bitmap_order_full_jenga_config():
    w = workloads.make_config(1)
    log(f"[order] {w.name}")
    d = to_dev(w)
    assert np.array_equal(gpu_order_bitmap(w, d), expected_order_bitmap(w))


@pytest.mark.parametrize("label,kw", BITMAP_CASES, ids=[c[0] for c in BITMAP_CASES])
def test_ordered_bitmap_forward_is_bitwise_the_unordered_one(label, kw):
    w = workloads.make_random(**kw)
    log(f"[order-fwd] bitmap {label}")
    d = to_dev(w)
    order = bsa.bsa_unit_order_bitmap(d["mask"], d["vbs"], B=w.B, H=w.H,
                                      S=w.S, Sk=w.Sk, block=w.block,
                                      mask_strides=w.mask_strides)
    ident = torch.arange(w.NQ, dtype=torch.int32, device="cuda").repeat(w.B * w.H)
    assert not torch.equal(order, ident)  # the ordered launch differs
    outs = []
    for qo in (None, order):
        out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        lse = torch.full((w.B, w.H, w.S), float("nan"), dtype=torch.float32,
                         device="cuda")
        bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                           block=w.block, sm_scale=w.sm_scale,
                           mask_strides=w.mask_strides, out=out, lse=lse,
                           balance=False, qblock_order=qo)
        torch.cuda.synchronize()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def test_bitmap_binding_orders_large_launches_by_default():
    """More units than run at once: the binding computes the order, and the
    result equals the q-block-order launch bit for bit."""
    w = workloads.make_random(324, B=1, H=20, S=64 * 64, block=64,
                              form="bitmap", density=0.5, vbs_mode="partial")
    assert bsa.api.launch_order_pays(w.B, w.H, w.NQ)
    log(f"[order-fwd] bitmap default order, {w.n_units} units")
    d = to_dev(w)
    a = run_gpu(w, dev_inputs=d)
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
    bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                       block=w.block, sm_scale=w.sm_scale,
                       mask_strides=w.mask_strides, out=out, lse=lse,
                       balance=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], out)
    assert torch.equal(a[1], lse)
