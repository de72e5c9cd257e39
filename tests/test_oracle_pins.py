"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against something it does not share code with:
library routines (torch's bf16/fp8 casts, torch SDPA, scipy logsumexp), an
independent dense brute force, closed forms and invariants of the definition
of sparse softmax attention (FastVideo "block_sparse_attn_sm100a.py",
`is_supported` docstring; rocke "sparse_attention.py", module docstring and
`_stage_vsa_bitmap_to_lds`; rocke "sage_attention.py", module docstring).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import bruteforce as bf

LOG2E = 1.0 / math.log(2.0)


def run_oracle(w, **kw):
    args = dict(block=w.block, sm_scale=w.sm_scale, k_scale=w.k_scale,
                v_scale=w.v_scale,
                k_codebook=w.k_codebook, v_codebook=w.v_codebook)
    args.update(kw)
    if w.form == "lut":
        return oracle.fwd_lut(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs,
                              meta_strides=w.meta_strides, **args)
    return oracle.fwd_bitmap(w.q, w.k, w.v, w.mask, w.vbs,
                             mask_strides=w.mask_strides, **args)


# ---------------------------------------------------------------- decoders

def test_bf16_decode_matches_torch_for_every_pattern():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b) & 0xFFFF) for b in bits.tolist()])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_fp8e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8e4m3_value(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert oracle.fp8e4m3_value(0x7E) == 448.0  # largest finite
    assert oracle.fp8e4m3_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert math.isnan(oracle.fp8e4m3_value(0x7F))


# ------------------------------------------------- dense reduction (SDPA)

@pytest.mark.parametrize("block,B,H,S", [(64, 2, 2, 256), (128, 1, 3, 512)])
def test_full_lut_equals_dense_sdpa(block, B, H, S):
    w = workloads.make_random(11 + block, B=B, H=H, S=S, block=block,
                              density=1.0)
    NQ = S // block
    assert int(w.q2k_num.min()) == NQ  # every block selected, vbs full
    o, lse = run_oracle(w)
    q = w.q.to(torch.float64)
    k = w.k.to(torch.float64)
    v = w.v.to(torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, scale=w.sm_scale).numpy()
    lse_ref = (torch.logsumexp(q @ k.transpose(-1, -2) * w.sm_scale, dim=-1)
               * LOG2E).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-10, rtol=1e-10)


def test_full_bitmap_equals_dense_sdpa_custom_scale():
    w = workloads.make_random(5, B=1, H=2, S=256, block=64, form="bitmap",
                              density=1.1)
    w.sm_scale = 0.37
    o, lse = run_oracle(w)
    q, k, v = (t.to(torch.float64) for t in (w.q, w.k, w.v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, scale=0.37).numpy()
    lse_ref = (torch.logsumexp(q @ k.transpose(-1, -2) * 0.37, dim=-1)
               * LOG2E).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-10, rtol=1e-10)


@pytest.mark.parametrize("H,Hk,S,Sk", [(4, 2, 256, 512), (3, 1, 512, 256),
                                       (2, 2, 128, 384)])
def test_rectangular_grouped_full_lut_equals_dense_sdpa(H, Hk, S, Sk):
    """Every key block selected with S_q != S_k and H query heads over Hk
    key/value heads reduces to dense attention with each K/V head repeated
    for its H/Hk query heads (rocke "sparse_attention.py": separate query
    and KV head counts and sequence lengths)."""
    w = workloads.make_random(60 + H + Sk // 64, B=2, H=H, S=S, block=64,
                              density=1.0, Hk=Hk, Sk=Sk)
    assert int(w.q2k_num.min()) == Sk // 64
    o, lse = run_oracle(w)
    q = w.q.to(torch.float64)
    k = w.k.to(torch.float64).repeat_interleave(H // Hk, dim=1).contiguous()
    v = w.v.to(torch.float64).repeat_interleave(H // Hk, dim=1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, scale=w.sm_scale).numpy()
    lse_ref = (torch.logsumexp(q @ k.transpose(-1, -2) * w.sm_scale, dim=-1)
               * LOG2E).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-10, rtol=1e-10)


def test_grouped_heads_equal_repeated_kv_heads():
    """GQA is the same computation as repeating each K/V head (and its fp8
    scales) for its query-head group: the oracle gives bitwise the same
    result both ways."""
    for kv in ("bf16", "fp8"):
        w = workloads.make_random(70, B=2, H=6, S=256, block=64, kv=kv,
                                  Hk=2, Sk=384, count_mode="uniform",
                                  vbs_mode="random")
        o, lse = run_oracle(w)
        def rep(t):
            return None if t is None else t.repeat_interleave(3, dim=1).contiguous()

        w2 = workloads.Workload(w.name, w.B, w.H, w.S, w.D, w.block, w.form,
                                w.q, rep(w.k), rep(w.v), k_scale=rep(w.k_scale),
                                v_scale=rep(w.v_scale), q2k_idx=w.q2k_idx,
                                q2k_num=w.q2k_num, meta_strides=w.meta_strides,
                                vbs=w.vbs, sm_scale=w.sm_scale)
        assert w2.Hk == w.H
        o2, l2 = run_oracle(w2)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2), kv


# ------------------------------------------------------ dense brute force

BRUTE_CASES = [
    dict(seed=1, block=64, S=256, density=0.5, vbs_mode="random"),
    dict(seed=2, block=64, S=512, count_mode="uniform", vbs_mode="zero_some"),
    dict(seed=3, block=128, S=512, count_mode="uniform", vbs_mode="partial",
         max_kv=3),
    dict(seed=4, block=64, S=256, form="bitmap", density=0.4,
         vbs_mode="random"),
    dict(seed=5, block=64, S=256, shared_meta=True, density=0.5,
         vbs_mode="partial"),
    dict(seed=6, block=64, S=256, form="bitmap", shared_meta=True,
         density=0.6),
    dict(seed=7, block=64, S=256, kv="fp8", density=0.5, vbs_mode="random"),
    dict(seed=8, block=128, S=256, kv="fp8", form="bitmap", density=0.7,
         std=3.0),
    dict(seed=9, block=64, S=256, Sk=448, H=4, Hk=2, count_mode="uniform",
         vbs_mode="zero_some"),
    dict(seed=10, block=64, S=384, Sk=192, H=3, Hk=1, form="bitmap",
         density=0.5, vbs_mode="partial"),
    dict(seed=11, block=128, S=256, Sk=512, H=4, Hk=1, kv="fp8",
         count_mode="uniform", vbs_mode="random"),
    dict(seed=12, block=64, S=256, kv="i8cb", density=0.5, vbs_mode="random"),
    dict(seed=13, block=64, S=256, kv="i4cb", form="bitmap", density=0.6,
         vbs_mode="partial"),
    dict(seed=14, block=128, S=256, Sk=512, H=4, Hk=2, kv="i4cb",
         count_mode="uniform"),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_dense_bruteforce(case):
    case = dict(case)
    seed = case.pop("seed")
    case.setdefault("H", 2)
    w = workloads.make_random(seed, B=2, **case)
    o, lse = run_oracle(w)
    o_ref, lse_ref = bf.attention(w)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-9)
    empty = lse_ref == bf.LSE_EMPTY
    assert (lse[empty] == bf.LSE_EMPTY).all()
    assert (o[empty] == 0).all()
    np.testing.assert_allclose(lse[~empty], lse_ref[~empty], atol=1e-10,
                               rtol=1e-10)


def test_units_subset_matches_full_run():
    w = workloads.make_random(9, B=2, H=3, S=512, block=64,
                              count_mode="uniform", vbs_mode="random")
    o, lse = run_oracle(w)
    units = [0, 5, 17, 47, 30]
    os_, ls_ = run_oracle(w, units=units)
    of = o.reshape(-1, w.block, w.D)
    lf = lse.reshape(-1, w.block)
    for i, u in enumerate(units):
        assert np.array_equal(os_[i], of[u])
        assert np.array_equal(ls_[i], lf[u])


# ------------------------------------------------------------ closed forms

def _single_row_lut(B, H, S, block, row_sets, vbs=None):
    """LUT workload with explicit per-unit sets (list of lists)."""
    NQ = S // block
    rows = B * H * NQ
    max_kv = max(1, max(len(s) for s in row_sets))
    idx = torch.full((rows, max_kv), -1, dtype=torch.int32)
    num = torch.zeros((rows,), dtype=torch.int32)
    for r, s in enumerate(row_sets):
        idx[r, :len(s)] = torch.tensor(s, dtype=torch.int32)
        num[r] = len(s)
    return idx, num


def test_zero_query_gives_mean_of_attended_values():
    w = workloads.make_random(21, B=1, H=2, S=256, block=64, density=0.5,
                              vbs_mode="partial")
    w.q = torch.zeros_like(w.q)
    o, lse = run_oracle(w)
    mask = bf.dense_mask(w)
    v = bf.to_f64(w.v)
    for h in range(w.H):
        for r in range(w.S):
            keys = np.nonzero(mask[0, h, r])[0]
            assert len(keys) > 0
            np.testing.assert_allclose(o[0, h, r], v[0, h, keys].mean(axis=0),
                                       atol=1e-12)
            assert abs(lse[0, h, r] - math.log2(len(keys))) < 1e-12


def test_single_attended_key_gives_its_value_and_score_lse():
    B, H, S, blk = 1, 1, 256, 64
    w = workloads.make_random(22, B=B, H=H, S=S, block=blk)
    # every q-block selects block 2 only; block 2 has exactly one valid key
    idx, num = _single_row_lut(B, H, S, blk, [[2]] * 4)
    w.q2k_idx, w.q2k_num = idx, num
    w.vbs = torch.tensor([64, 64, 1, 64], dtype=torch.int32)
    o, lse = run_oracle(w)
    q = bf.to_f64(w.q)[0, 0]
    k = bf.to_f64(w.k)[0, 0, 128]
    v = bf.to_f64(w.v)[0, 0, 128]
    for r in range(S):
        np.testing.assert_array_equal(o[0, 0, r], v)
        t = float(q[r] @ k) * w.sm_scale * LOG2E
        assert abs(lse[0, 0, r] - t) < 1e-11


def test_two_keys_give_sigmoid_weights():
    B, H, S, blk = 1, 1, 128, 64
    w = workloads.make_random(23, B=B, H=H, S=S, block=blk)
    idx, num = _single_row_lut(B, H, S, blk, [[1], [0]])
    w.q2k_idx, w.q2k_num = idx, num
    w.vbs = torch.tensor([2, 2], dtype=torch.int32)
    o, lse = run_oracle(w)
    q = bf.to_f64(w.q)[0, 0]
    k = bf.to_f64(w.k)[0, 0]
    v = bf.to_f64(w.v)[0, 0]
    for r in range(S):
        kb = 1 if r < 64 else 0
        k0, k1 = k[kb * 64], k[kb * 64 + 1]
        a = q[r] @ k0 * w.sm_scale
        b = q[r] @ k1 * w.sm_scale
        w0 = 1.0 / (1.0 + math.exp(b - a))
        np.testing.assert_allclose(
            o[0, 0, r], w0 * v[kb * 64] + (1 - w0) * v[kb * 64 + 1],
            atol=1e-12, rtol=1e-12)
        ref = (max(a, b) + math.log1p(math.exp(-abs(a - b)))) * LOG2E
        assert abs(lse[0, 0, r] - ref) < 1e-12


def test_count_zero_rows_give_exact_zero_and_sentinel():
    w = workloads.make_random(24, B=1, H=2, S=256, block=64,
                              count_mode="zero")
    o, lse = run_oracle(w)
    assert (o == 0).all() and not np.signbit(o).any()
    assert (lse == oracle.LSE_EMPTY).all()
    assert oracle.LSE_EMPTY == -3.4028234663852886e38


def test_all_selected_blocks_empty_by_vbs_is_an_empty_row():
    w = workloads.make_random(25, B=1, H=1, S=256, block=64, density=0.5)
    w.vbs = torch.zeros((4,), dtype=torch.int32)
    o, lse = run_oracle(w)
    assert (o == 0).all() and (lse == oracle.LSE_EMPTY).all()


# -------------------------------------------------------------- invariants

def _lut_copy(w, idx=None, num=None):
    import copy
    w2 = copy.copy(w)
    if idx is not None:
        w2.q2k_idx = idx
    if num is not None:
        w2.q2k_num = num
    return w2


def test_lut_order_padding_and_duplicates_do_not_matter():
    w = workloads.make_random(31, B=2, H=2, S=512, block=64, max_kv=6,
                              count_mode="uniform", vbs_mode="random")
    o, lse = run_oracle(w)
    g = torch.Generator().manual_seed(0)
    idx = w.q2k_idx.clone()
    num = w.q2k_num
    for r in range(idx.shape[0]):
        n = int(num[r])
        idx[r, :n] = idx[r, :n][torch.randperm(n, generator=g)]
        pads = torch.tensor([-2**31, w.NQ + 5, 10**6, -1, w.NQ, 7],
                            dtype=torch.int32)
        idx[r, n:] = pads[:idx.shape[1] - n]
    o2, l2 = run_oracle(_lut_copy(w, idx=idx))
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # duplicates: append each row's first entry again in a wider LUT
    wide = torch.full((idx.shape[0], idx.shape[1] + 1), -1, dtype=torch.int32)
    num2 = num.clone()
    for r in range(idx.shape[0]):
        n = int(num[r])
        wide[r, :n] = idx[r, :n]
        if n > 0:
            wide[r, n] = idx[r, 0]
            num2[r] = n + 1
    o3, l3 = run_oracle(_lut_copy(w, idx=wide, num=num2))
    assert np.array_equal(o, o3) and np.array_equal(lse, l3)


def test_out_of_range_entries_and_counts_are_skipped_and_clamped():
    w = workloads.make_random(32, B=1, H=2, S=256, block=64, max_kv=4,
                              count_mode="uniform")
    o, lse = run_oracle(w)
    idx = w.q2k_idx.clone()
    num = w.q2k_num.clone()
    # insert an out-of-range entry below the count (skipped) by widening
    wide = torch.full((idx.shape[0], 6), 3, dtype=torch.int32)
    num2 = num.clone()
    for r in range(idx.shape[0]):
        n = int(num[r])
        row = idx[r, :n].tolist() + [w.NQ + 3]
        wide[r, :len(row)] = torch.tensor(row, dtype=torch.int32)
        num2[r] = len(row)
    o2, l2 = run_oracle(_lut_copy(w, idx=wide, num=num2))
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # count above max_kv is clamped to max_kv; negative count means 0
    full = _lut_copy(w, num=torch.full_like(num, 4))
    o3, l3 = run_oracle(full)
    o4, l4 = run_oracle(_lut_copy(w, num=torch.full_like(num, 99)))
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    o5, l5 = run_oracle(_lut_copy(w, num=torch.full_like(num, -7)))
    assert (o5 == 0).all() and (l5 == oracle.LSE_EMPTY).all()


def test_vbs_is_clamped_to_block():
    w = workloads.make_random(33, B=1, H=1, S=256, block=64, density=0.5)
    o, lse = run_oracle(w)
    w.vbs = torch.tensor([64, 1000, 64, 65], dtype=torch.int32)
    o2, l2 = run_oracle(w)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_bitmap_equals_compacted_lut():
    w = workloads.make_random(34, B=2, H=2, S=512, block=64, form="bitmap",
                              density=0.4, vbs_mode="random")
    o, lse = run_oracle(w)
    # compaction by numpy (independent of the oracle's own compaction)
    m = w.mask.numpy()
    idx = np.full(m.shape, -1, dtype=np.int32)
    num = np.zeros(m.shape[0], dtype=np.int32)
    for r in range(m.shape[0]):
        nz = np.nonzero(m[r])[0]
        idx[r, :len(nz)] = nz
        num[r] = len(nz)
    o2, l2 = oracle.fwd_lut(w.q, w.k, w.v, torch.from_numpy(idx),
                            torch.from_numpy(num), w.vbs, block=w.block,
                            meta_strides=w.mask_strides)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    i3, n3 = oracle.mask_to_lut(w.mask)
    assert np.array_equal(i3.numpy(), idx) and np.array_equal(n3.numpy(), num)


def test_output_is_linear_in_v():
    w = workloads.make_random(35, B=1, H=2, S=256, block=64, density=0.5,
                              vbs_mode="partial")
    o, lse = run_oracle(w)
    w.v = (-2.0 * w.v.float()).to(torch.bfloat16)  # exact in bf16
    o2, l2 = run_oracle(w)
    np.testing.assert_allclose(o2, -2.0 * o, atol=1e-12, rtol=1e-12)
    assert np.array_equal(lse, l2)


def test_common_key_shift_moves_lse_only():
    """Adding one vector u to every key multiplies every weight of a row by
    2^(c q.u): O is unchanged and LSE shifts by c*q.u (integer data so that
    K + u is exact in bf16)."""
    g = torch.Generator().manual_seed(36)
    w = workloads.make_random(36, B=1, H=1, S=256, block=64, density=0.5,
                              vbs_mode="partial")
    w.q = torch.randint(-3, 4, w.q.shape, generator=g).to(torch.bfloat16)
    w.k = torch.randint(-3, 4, w.k.shape, generator=g).to(torch.bfloat16)
    o, lse = run_oracle(w)
    u = torch.randint(-2, 3, (w.D,), generator=g)
    w2 = _lut_copy(w)
    w2.k = (w.k.float() + u.float()).to(torch.bfloat16)
    o2, l2 = run_oracle(w2)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=1e-10)
    shift = (w.q.double() @ u.double()).numpy() * w.sm_scale * LOG2E
    np.testing.assert_allclose(l2, lse + shift, atol=1e-10)


def test_heads_and_batches_are_independent():
    w = workloads.make_random(37, B=2, H=3, S=256, block=64,
                              count_mode="uniform", vbs_mode="random")
    o, lse = run_oracle(w)
    NQ = w.NQ
    for b in range(w.B):
        for h in range(w.H):
            rows = slice((b * w.H + h) * NQ, (b * w.H + h + 1) * NQ)
            o1, l1 = oracle.fwd_lut(
                w.q[b:b + 1, h:h + 1], w.k[b:b + 1, h:h + 1],
                w.v[b:b + 1, h:h + 1], w.q2k_idx[rows], w.q2k_num[rows],
                w.vbs, block=w.block, meta_strides=(NQ, NQ))
            assert np.array_equal(o1[0, 0], o[b, h])
            assert np.array_equal(l1[0, 0], lse[b, h])


def test_fp8_scales_fold_linearly():
    """Doubling V's block scales doubles O; doubling K's scale doubles every
    logit (checked against the brute force)."""
    w = workloads.make_random(38, B=1, H=2, S=256, block=64, kv="fp8",
                              density=0.5)
    o, lse = run_oracle(w)
    w.v_scale = w.v_scale * 2
    o2, l2 = run_oracle(w)
    np.testing.assert_allclose(o2, 2 * o, atol=1e-12, rtol=1e-12)
    assert np.array_equal(l2, lse)
    w.k_scale = w.k_scale * 2
    o3, l3 = run_oracle(w)
    o_ref, l_ref = bf.attention(w)
    np.testing.assert_allclose(o3, o_ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(l3, l_ref, atol=1e-10)


# ---------------------------------------------------- integer decode only

@pytest.mark.parametrize("form,Sk", [("lut", None), ("bitmap", None),
                                     ("lut", 832), ("bitmap", 192)])
def test_key_counts_match_python_sets(form, Sk):
    w = workloads.make_random(41, B=2, H=2, S=512, block=64, form=form,
                              count_mode="uniform", density=0.3,
                              vbs_mode="random", Sk=Sk)
    kw = dict(B=w.B, H=w.H, S=w.S, Sk=w.Sk, block=w.block, vbs=w.vbs)
    if form == "lut":
        c = oracle.key_counts(q2k_idx=w.q2k_idx, q2k_num=w.q2k_num,
                              meta_strides=w.meta_strides, **kw)
    else:
        c = oracle.key_counts(mask=w.mask, mask_strides=w.mask_strides, **kw)
    sets = bf.selected_sets(w)
    vbs = w.vbs.tolist()
    for u, s in enumerate(sets):
        want = [min(max(vbs[kb], 0), w.block) if kb in s else 0
                for kb in range(w.NK)]
        assert c[u].tolist() == want


def test_tiny_named_workload_runs_and_has_expected_structure():
    w = workloads.make_config(0)
    assert (w.B, w.H, w.S, w.block) == (1, 1, 512, 64)
    assert w.vbs.tolist() == [64] * 7 + [40]
    assert (w.q2k_num == 4).all()
    o, lse = run_oracle(w)
    o_ref, l_ref = bf.attention(w)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(lse, l_ref, atol=1e-10)


# ------------------------------------------------------------- backward

def _dout(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.q.shape, generator=g).to(torch.bfloat16)


def _oracle_bwd(w, dout):
    kw = dict(block=w.block, vbs=w.vbs, sm_scale=w.sm_scale)
    if w.form == "lut":
        return oracle.bwd(w.q, w.k, w.v, dout, q2k_idx=w.q2k_idx,
                          q2k_num=w.q2k_num, meta_strides=w.meta_strides, **kw)
    return oracle.bwd(w.q, w.k, w.v, dout, mask=w.mask,
                      meta_strides=w.mask_strides, **kw)


@pytest.mark.parametrize("H,Hk,S,Sk", [(2, 2, 256, 256), (4, 2, 128, 384)])
def test_backward_full_selection_equals_sdpa_autograd(H, Hk, S, Sk):
    """Every block selected: the oracle's gradients equal torch autograd
    through SDPA in float64 (a library routine), K/V heads repeated per
    group (autograd sums their gradients)."""
    w = workloads.make_random(80 + H, B=2, H=H, Hk=Hk, S=S, Sk=Sk, block=64,
                              density=1.0)
    dout = _dout(w, 1)
    dq, dk, dv = _oracle_bwd(w, dout)
    q = w.q.to(torch.float64).requires_grad_(True)
    k = w.k.to(torch.float64).requires_grad_(True)
    v = w.v.to(torch.float64).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(H // Hk, dim=1),
        v.repeat_interleave(H // Hk, dim=1), scale=w.sm_scale)
    (o * dout.to(torch.float64)).sum().backward()
    for got, ref in ((dq, q.grad), (dk, k.grad), (dv, v.grad)):
        np.testing.assert_allclose(got, ref.numpy(), atol=1e-10, rtol=1e-9)


BWD_CASES = [
    dict(seed=91, block=64, S=256, count_mode="uniform", vbs_mode="zero_some"),
    dict(seed=92, block=64, S=256, form="bitmap", density=0.4,
         vbs_mode="random"),
    dict(seed=93, block=128, S=256, Sk=512, H=4, Hk=2, count_mode="uniform",
         vbs_mode="partial"),
    dict(seed=94, block=64, S=192, Sk=128, H=3, Hk=1, shared_meta=True,
         density=0.5, vbs_mode="partial"),
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_dense_autograd(case):
    """Sparse selections, ragged blocks, empty rows, grouped heads and
    S_q != S_k: the oracle's hand-derived chain rule against torch autograd
    through an independent dense masked softmax."""
    case = dict(case)
    seed = case.pop("seed")
    case.setdefault("H", 2)
    w = workloads.make_random(seed, B=2, **case)
    dout = _dout(w, seed)
    dq, dk, dv = _oracle_bwd(w, dout)
    rq, rk, rv = bf.grads_autograd(w, dout)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, atol=1e-10, rtol=1e-9)


def test_backward_empty_rows_have_zero_dq_and_no_kv_gradient():
    w = workloads.make_random(95, B=1, H=2, S=256, block=64,
                              count_mode="zero")
    dq, dk, dv = _oracle_bwd(w, _dout(w, 3))
    assert not dq.any() and not dk.any() and not dv.any()


def test_backward_is_linear_in_dout_and_dv_is_p_transpose_dout():
    """dq, dk, dv are linear in dout; with dout = 0 all vanish."""
    w = workloads.make_random(96, B=1, H=2, S=256, block=64, density=0.5,
                              vbs_mode="partial")
    d1 = _dout(w, 5)
    g1 = _oracle_bwd(w, d1)
    d2 = (-2.0 * d1.float()).to(torch.bfloat16)  # exact in bf16
    g2 = _oracle_bwd(w, d2)
    for a_, b_ in zip(g1, g2):
        np.testing.assert_allclose(b_, -2.0 * a_, atol=1e-12, rtol=1e-12)
    g0 = _oracle_bwd(w, torch.zeros_like(d1))
    assert all(not x.any() for x in g0)


# ------------------------------------------------------- codebook K/V

def test_codebook_index_worked_example():
    """i8: level = code + 128.  i4: two codes per byte, element 2i in the
    low nibble, two's complement, level = code + 8 (rocke
    "sage_attention.py", codebook-dequant primitives)."""
    i8 = torch.tensor([-128, -1, 0, 127], dtype=torch.int8)
    assert [oracle.codebook_index(oracle.KV_I8_CODEBOOK, i8, e)
            for e in range(4)] == [0, 127, 128, 255]
    i4 = torch.tensor([0x9F, 0x70], dtype=torch.uint8)
    # 0x9F: low 0xF = -1 -> 7, high 0x9 = -7 -> 1; 0x70: low 0 -> 8, high 7 -> 15
    assert [oracle.codebook_index(oracle.KV_I4_CODEBOOK, i4, e)
            for e in range(4)] == [7, 1, 8, 15]


def test_integer_codebook_equals_bf16_values():
    """An integer codebook with unit scales is the same attention as bf16
    K/V holding those integers: bitwise equal oracle results."""
    w = workloads.make_random(97, B=1, H=2, S=256, block=64, kv="i8cb",
                              density=0.5, vbs_mode="partial")
    w.k_codebook = torch.arange(-128, 128, dtype=torch.float32) / 16.0
    w.v_codebook = torch.arange(-128, 128, dtype=torch.float32) / 32.0
    w.k_scale = torch.ones_like(w.k_scale)
    w.v_scale = torch.ones_like(w.v_scale)
    o, lse = run_oracle(w)
    kb = torch.from_numpy(bf.codebook_values(w.k, w.k_codebook)).to(torch.bfloat16)
    vb = torch.from_numpy(bf.codebook_values(w.v, w.v_codebook)).to(torch.bfloat16)
    o2, l2 = oracle.fwd_lut(w.q, kb, vb, w.q2k_idx, w.q2k_num, w.vbs,
                            block=w.block, meta_strides=w.meta_strides)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


# ------------------------------------------- the softmax scale's full domain

def test_oracle_rejects_a_non_finite_softmax_scale():
    w = workloads.make_random(60, B=1, H=1, S=128, block=64)
    for bad in (float("nan"), float("inf"), -float("inf")):
        with pytest.raises(ValueError):
            run_oracle(w, sm_scale=bad)
    with pytest.raises(ValueError):
        oracle.bwd(w.q, w.k, w.v, w.q, block=64, q2k_idx=w.q2k_idx,
                   q2k_num=w.q2k_num, sm_scale=float("nan"))


SCALE_CASES = [
    dict(seed=61, sm_scale=0.37, vbs_mode="partial"),
    dict(seed=62, sm_scale=2.0, vbs_mode="random", form="bitmap"),
    dict(seed=63, sm_scale=0.0, vbs_mode="partial", count_mode="uniform"),
    dict(seed=64, sm_scale=-0.5, vbs_mode="zero_some", block=128, S=512),
    dict(seed=65, sm_scale=-1.25, kv="fp8", vbs_mode="partial"),
]


@pytest.mark.parametrize("case", SCALE_CASES)
def test_any_finite_softmax_scale_matches_dense_bruteforce(case):
    case = dict(case)
    seed, scale = case.pop("seed"), case.pop("sm_scale")
    case.setdefault("S", 256)
    case.setdefault("block", 64)
    case.setdefault("density", 0.5)
    w = workloads.make_random(seed, B=1, H=2, **case)
    w.sm_scale = scale
    o, lse = run_oracle(w)
    o_ref, l_ref = bf.attention(w)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-9)
    empty = l_ref == bf.LSE_EMPTY
    assert (lse[empty] == bf.LSE_EMPTY).all()
    np.testing.assert_allclose(lse[~empty], l_ref[~empty], atol=1e-10,
                               rtol=1e-10)


def test_zero_softmax_scale_gives_mean_of_attended_values():
    """sm_scale = 0: every attended key has weight 1, so O is the plain mean
    of the attended values and LSE = log2(number of attended keys)."""
    w = workloads.make_random(66, B=1, H=2, S=256, block=64, density=0.5,
                              vbs_mode="partial")
    w.sm_scale = 0.0
    o, lse = run_oracle(w)
    mask = bf.dense_mask(w)
    v = bf.to_f64(w.v)
    for h in range(w.H):
        for r in range(w.S):
            keys = np.nonzero(mask[0, h, r])[0]
            np.testing.assert_allclose(o[0, h, r], v[0, h, keys].mean(axis=0),
                                       atol=1e-12)
            assert lse[0, h, r] == math.log2(len(keys))


def test_negative_softmax_scale_equals_negated_query():
    """t = (q . k) * c: negating the scale is negating every query (exact in
    bf16 and in the products)."""
    w = workloads.make_random(67, B=1, H=2, S=256, block=64, density=0.5,
                              vbs_mode="random")
    w.sm_scale = -0.3
    o, lse = run_oracle(w)
    w.sm_scale = 0.3
    w.q = -w.q
    o2, l2 = run_oracle(w)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_zero_and_negative_fp8_block_scales_are_exact_products():
    """A key block whose K scale is 0 scores exactly 0 on every query; a
    block whose V scale is 0 contributes zero values but keeps its weights;
    a negative scale negates the block (each against the dense brute force,
    whose decode is torch's fp8 cast times the scale)."""
    w = workloads.make_random(68, B=1, H=2, S=512, block=64, kv="fp8",
                              density=0.6, vbs_mode="partial")
    ks, vs = w.k_scale.clone(), w.v_scale.clone()
    k = w.k.clone()
    k[:, :, 64:128] = torch.zeros((1, 2, 64, 128)).to(torch.float8_e4m3fn)
    ks[:, :, 1] = 0.0              # the all-zero block of amax/448 = 0
    ks[:, 0, 3] = 0.0              # nonzero codes, zero scale
    vs[:, 1, 2] = 0.0
    ks[:, 1, 5] = -ks[:, 1, 5]
    vs[:, 0, 6] = -2.0 * vs[:, 0, 6]
    w.k, w.k_scale, w.v_scale = k, ks, vs
    o, lse = run_oracle(w)
    o_ref, l_ref = bf.attention(w)
    np.testing.assert_allclose(o, o_ref, atol=1e-10, rtol=1e-9)
    np.testing.assert_allclose(lse, l_ref, atol=1e-10, rtol=1e-10)
