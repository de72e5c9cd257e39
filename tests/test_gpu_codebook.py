"""Codebook K/V on the GPU: bsa_codebook_dequant bit-exact against torch
indexing of the bf16-rounded codebook, and the forward pass on
codebook-coded K/V (dequantisation + BSA_KV_BF16_SCALED) against the
oracle's codebook modes."""

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
import oracle
from tests.gpu_helpers import check, log, run_oracle, scaled_input_bounds

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def levels(codes: torch.Tensor) -> torch.Tensor:
    """Codebook levels by numpy (i8: code + 128; i4: nibbles, low first)."""
    c = codes.numpy()
    if c.dtype == np.int8:
        return torch.from_numpy(c.astype(np.int64) + 128)
    lo = (c & 15).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    lv = np.stack([np.where(lo >= 8, lo - 16, lo), np.where(hi >= 8, hi - 16, hi)],
                  axis=-1).reshape(*c.shape[:-1], 2 * c.shape[-1]) + 8
    return torch.from_numpy(lv)


@pytest.mark.parametrize("kind,n", [("i8", 16), ("i8", 4096 * 48), ("i4", 16),
                                    ("i4", 4096 * 32), ("i8", 0),
                                    # ragged: the last workgroup is partial
                                    ("i8", 16 * 12345), ("i4", 16 * 9999)])
def test_dequant_bit_exact(kind, n):
    g = torch.Generator().manual_seed(n + len(kind))
    ent = 256 if kind == "i8" else 16
    cb = torch.randn((ent,), generator=g) * 3.0  # not bf16-exact: RNE path
    if kind == "i8":
        codes = torch.randint(-128, 128, (n,), generator=g, dtype=torch.int8)
    else:
        codes = torch.randint(0, 256, (n // 2,), generator=g,
                              dtype=torch.int32).to(torch.uint8)
    log(f"[dequant] {kind} n={n}")
    got = bsa.bsa_codebook_dequant(codes.cuda(), cb.cuda())
    torch.cuda.synchronize()
    ref = cb.to(torch.bfloat16)[levels(codes)]
    assert got.shape == ref.shape
    assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))


CASES = [
    ("i8_lut64", dict(seed=401, B=1, H=2, S=512, block=64, kv="i8cb",
                      density=0.5, vbs_mode="partial")),
    ("i4_lut64_uniform", dict(seed=402, B=2, H=2, S=512, block=64, kv="i4cb",
                              count_mode="uniform", vbs_mode="random")),
    ("i4_bitmap128", dict(seed=403, B=1, H=2, S=1024, block=128, kv="i4cb",
                          form="bitmap", density=0.4)),
    ("i8_gqa_rect", dict(seed=404, B=1, H=4, Hk=2, S=512, Sk=768, block=64,
                         kv="i8cb", count_mode="uniform", vbs_mode="zero_some")),
    ("i4_gqa128", dict(seed=405, B=1, H=6, Hk=3, S=512, Sk=1024, block=128,
                       kv="i4cb", density=0.5, vbs_mode="partial")),
]


def vmax(w) -> float:
    """Largest dequantised |V| (codebook level times block scale): the
    codebook levels span each block's range, so the bound derived for
    inputs beyond N(0, 1) applies (P rounded to bf16 moves O by at most
    2^-9 max|V|)."""
    return float(w.v_codebook.abs().max() * w.v_scale.max())


def run_codebook_gpu(w):
    d = {n: (None if getattr(w, n) is None else getattr(w, n).cuda())
         for n in ("q", "k", "v", "k_scale", "v_scale", "q2k_idx", "q2k_num",
                   "mask", "vbs", "k_codebook", "v_codebook")}
    out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((w.B, w.H, w.S), float("nan"), dtype=torch.float32,
                     device="cuda")
    kw = dict(block=w.block, sm_scale=w.sm_scale, k_scale=d["k_scale"],
              v_scale=d["v_scale"], k_codebook=d["k_codebook"],
              v_codebook=d["v_codebook"], out=out, lse=lse)
    if w.form == "lut":
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        d["vbs"], meta_strides=w.meta_strides, **kw)
    else:
        bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                           mask_strides=w.mask_strides, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_codebook_forward_parity(label, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    log(f"[codebook fwd] {label} {w.k.dtype} B{w.B} H{w.H} Hk{w.Hk} S{w.S} "
        f"Sk{w.Sk} blk{w.block}")
    out, lse = run_codebook_gpu(w)
    o_ref, l_ref = run_oracle(w)
    o_abs, o_rel = scaled_input_bounds(vmax(w))
    check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, label,
          o_rel=o_rel, o_abs=o_abs)


def codebook_rounding_bounds(w):
    """Per query row r, the bound E_r on how far bf16 operands move the
    scores t from the oracle's f32-table values.  The products run on bf16
    operands (the rocke sage page's is_valid_spec: every path ends in the
    f16/bf16 QK/PV atom), so each K and V value is codebook[level] rounded
    to bf16 (RNE: relative error <= 2^-9) times its block scale.  Then
    |t'_rj - t_rj| <= |c| 2^-9 sum_d |q_rd| |k_jd| <= E_r over the row's
    attended keys j, and
      |LSE'_r - LSE_r| = |log2(sum_j 2^t'_rj / sum_j 2^t_rj)| <= E_r,
      |O'_r - O_r| <= (2^(2 E_r) - 1) max|v| + 2^-9 max|v|
    (each normalised weight moves by a factor within 2^(+-2 E_r); each value
    by at most 2^-9 of itself).  Returns (E [B,H,S], max|v|)."""
    from tests import bruteforce as bf
    mask = bf.dense_mask(w)
    q = np.abs(bf.to_f64(w.q))
    k, v = bf.kv_f64(w)
    c = abs(w.sm_scale) / np.log(2.0)
    s = np.einsum("bhsd,bhtd->bhst", q, np.abs(k)) * c * 2.0 ** -9
    e = np.where(mask, s, 0.0).max(axis=-1)
    return e, float(np.abs(v).max())


def test_codebook_not_bf16_exact_within_derived_bound():
    """An fp32 codebook that bf16 cannot hold: the GPU result (bf16 operands)
    against the oracle on the f32 table itself, within the bound that the
    codebook's rounding to bf16 allows (codebook_rounding_bounds) on top of
    the kernel's own bound."""
    w = workloads.make_random(406, B=1, H=2, S=512, block=64, kv="i8cb",
                              density=0.5, vbs_mode="partial")
    g = torch.Generator().manual_seed(9)
    w.k_codebook = (w.k_codebook + torch.randn(256, generator=g) * 1e-3)
    w.v_codebook = (w.v_codebook + torch.randn(256, generator=g) * 1e-3)
    assert not torch.equal(w.k_codebook.to(torch.bfloat16).float(), w.k_codebook)
    log("[codebook fwd] fp32 codebook, oracle on the f32 table")
    out, lse = run_codebook_gpu(w)
    o_ref, l_ref = run_oracle(w)
    e, v_max = codebook_rounding_bounds(w)
    o_abs, o_rel = scaled_input_bounds(v_max)
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    l_gpu = lse.cpu().numpy().astype(np.float64)
    o_ref = o_ref.reshape(o_gpu.shape)
    l_ref = l_ref.reshape(l_gpu.shape)
    empty = l_ref == oracle.LSE_EMPTY
    assert (l_gpu[empty] == l_ref[empty]).all()
    assert (o_gpu[empty] == 0).all()
    ne = ~empty
    lse_bound = 1e-3 + e
    err_l = np.abs(l_gpu - l_ref)
    o_bound = (o_abs + o_rel * np.abs(o_ref)
               + ((np.exp2(2.0 * e) - 1.0) * v_max + 2.0 ** -9 * v_max)[..., None])
    err_o = np.abs(o_gpu - o_ref)
    log(f"  max dLSE {err_l[ne].max():.3e} (bound {lse_bound[ne].max():.3e}), "
        f"max dO {err_o.max():.3e}, largest E {e.max():.3e}")
    assert (err_l[ne] <= lse_bound[ne]).all()
    assert (err_o <= o_bound).all()
