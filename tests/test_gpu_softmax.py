"""GPU parity of the softmax step over the whole domain of the scales.

The forward kernel first runs every unit with a fixed per-row reference (the
first tile's row maximum, taken over t = s*c) and recomputes a unit with the
online running-max rescale when a weight or a row sum overflowed.  These
cases check, against the oracle:
  - softmax scales other than 1/sqrt(D): 0.37, 2, 0 (equal weights),
    negative (reversed ranking), with keys masked by variable_block_sizes;
  - fp8 key blocks whose scale is 0 (an all-zero block quantised with
    amax/448), zero V scales and negative scales;
  - workloads whose later keys score more than 2^7 log2 units above the
    first tile's maximum, so that the rescaling pass must run (the test
    asserts from the inputs, on the CPU, that such rows exist).
Tolerances: LSE 1e-3 (the target's).  O: the bound derived from the
kernel's two bf16 roundings, 1e-2 + 2^-8 |O| + 2^-9 max|V| -- the target's
1e-2 is stated for N(0, 1) inputs at the default scale 1/sqrt(D); a sharper
softmax (larger |scale|, or a planted block that dominates) puts O near a
single V row, where |O| reaches ~3-4 and the bf16 output spacing alone is
2^-6, and the probabilities' rounding to bf16 moves O by up to
2^-9 max|V|."""

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from tests import bruteforce as bf
from tests.gpu_helpers import (check, gather_units, log, run_gpu, run_oracle,
                               scaled_input_bounds)

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _units(w, n=48):
    if w.n_units <= n:
        return None
    return sorted(set(np.linspace(0, w.n_units - 1, n).astype(int).tolist()))


def _parity(w, label):
    out, lse = run_gpu(w)
    units = _units(w)
    o_ref, l_ref = run_oracle(w, units=units)
    if units is None:
        o_gpu, l_gpu = out.float().cpu().numpy(), lse.cpu().numpy()
        o_ref = o_ref.reshape(o_gpu.shape)
        l_ref = l_ref.reshape(l_gpu.shape)
    else:
        o_gpu, l_gpu = gather_units(w, out, lse, units)
    v_max = float(np.abs(bf.kv_f64(w)[1]).max())  # decoded values
    o_abs, o_rel = scaled_input_bounds(v_max)
    check(o_gpu, l_gpu, o_ref, l_ref, label, o_rel=o_rel, o_abs=o_abs)
    assert torch.isfinite(out.float()).all().item()
    return o_ref, l_ref


SCALES = [
    ("lut64_scale_0.37", 0.37, dict(seed=301, B=1, H=2, S=1024, block=64,
                                    density=0.5, vbs_mode="partial")),
    ("lut64_scale_2", 2.0, dict(seed=302, B=1, H=2, S=1024, block=64,
                                count_mode="uniform", vbs_mode="edges")),
    ("bitmap128_scale_0", 0.0, dict(seed=303, B=1, H=2, S=1024, block=128,
                                    form="bitmap", density=0.4,
                                    vbs_mode="edges")),
    ("lut64_scale_neg", -0.5, dict(seed=304, B=1, H=2, S=2048, block=64,
                                   density=0.7, vbs_mode="tiny")),
    ("lut128_scale_neg", -0.2, dict(seed=305, B=2, H=1, S=1024, block=128,
                                    count_mode="uniform",
                                    vbs_mode="zero_some")),
    ("fp8_lut64_scale_neg", -1.25, dict(seed=306, B=1, H=2, S=1024, block=64,
                                        kv="fp8", density=0.5,
                                        vbs_mode="partial")),
    ("fp8_bitmap128_scale_0", 0.0, dict(seed=307, B=1, H=2, S=1024,
                                        block=128, kv="fp8", form="bitmap",
                                        density=0.5, vbs_mode="partial")),
    ("scaled_bf16_lut64_scale_2", 2.0, dict(seed=308, B=1, H=2, S=1024,
                                            block=64, kv="i8cb", density=0.5,
                                            vbs_mode="partial")),
]


@pytest.mark.parametrize("label,scale,kw", SCALES, ids=[c[0] for c in SCALES])
def test_softmax_scale_domain_parity(label, scale, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    w.sm_scale = scale
    log(f"[softmax] {label} sm_scale={scale} blk{w.block} form={w.form}")
    _parity(w, label)


def test_fp8_zero_and_negative_block_scales_parity():
    """Zero K scale (an all-zero block, and a block of nonzero codes), zero V
    scale, negative K and V scales, with partial blocks so that masked keys
    sit in tiles whose score scale is 0 or negative."""
    w = workloads.make_random(310, B=1, H=2, S=1024, block=64, kv="fp8",
                              density=0.6, vbs_mode="partial")
    k, ks, vs = w.k.clone(), w.k_scale.clone(), w.v_scale.clone()
    k[:, :, 64:128] = torch.zeros((1, 2, 64, 128)).to(torch.float8_e4m3fn)
    ks[:, :, 1] = 0.0
    ks[:, 0, 3] = 0.0
    ks[:, :, 0] = 0.0      # the lowest block: the first tile's scale is 0
    vs[:, 1, 2] = 0.0
    ks[:, 1, 5] = -ks[:, 1, 5]
    ks[:, :, 9:12] = -ks[:, :, 9:12]
    vs[:, 0, 6] = -2.0 * vs[:, 0, 6]
    w.k, w.k_scale, w.v_scale = k, ks, vs
    log("[softmax] fp8 zero / negative block scales")
    _parity(w, "fp8_zero_neg_scales")


def _key_groups(w, keys):
    """A unit's attended keys (ascending) as its wave groups sweep them.  A
    split launch (block 64, bf16 K/V, at most BSA_FWD_KEY_SPLIT_MAX_UNITS
    units) hands the selected blocks up to the first one at which the
    running count of valid keys reaches half the unit's total (at least one
    block) to group 0 and the rest to group 1; otherwise one group takes
    them all.  Each group starts its own fixed reference."""
    split = (w.block == 64 and not (w.kv_fp8 or w.kv_codebook)
             and w.n_units <= bsa.BSA_FWD_KEY_SPLIT_MAX_UNITS)
    if not split:
        return [keys]
    _, counts = np.unique(keys // w.block, return_counts=True)
    cum = np.cumsum(counts)
    e1 = min(max(int(np.argmax(2 * cum >= cum[-1])) + 1, 1), len(counts))
    cut = int(cum[e1 - 1])
    return [g for g in (keys[:cut], keys[cut:]) if len(g)]


def _rescale_gaps(w, units):
    """Per checked unit, the largest gap over its rows and wave groups
    between the group's log2-sum of weights, log2 sum 2^t, and the group's
    fixed reference: the maximum of t over the group's first tile (the first
    32 keys of its stream of valid keys for bf16 K/V; the lowest block's
    first min(32, valid) keys when K/V carry per-block scales), by dense
    float64 arithmetic.  None for a unit without keys."""
    mask = bf.dense_mask(w)
    q = bf.to_f64(w.q)
    k, _ = bf.kv_f64(w)
    c = w.sm_scale * LOG2E
    per_block = w.kv_fp8 or w.kv_codebook
    res = []
    for u in units:
        qb = u % w.NQ
        h = (u // w.NQ) % w.H
        b = u // (w.NQ * w.H)
        rows = slice(qb * w.block, (qb + 1) * w.block)
        keys = np.nonzero(mask[b, h, qb * w.block])[0]
        if len(keys) == 0:
            res.append(None)
            continue
        gap = -np.inf
        for grp in _key_groups(w, keys):
            if per_block:
                first = grp[grp // w.block == grp[0] // w.block][:32]
            else:
                first = grp[:32]
            m = (q[b, h, rows] @ k[b, h, first].T * c).max(axis=1)
            t = q[b, h, rows] @ k[b, h, grp].T * c
            tm = t.max(axis=1)
            lsum = tm + np.log2(np.exp2(t - tm[:, None]).sum(axis=1))
            gap = max(gap, float((lsum - m).max()))
        res.append(gap)
    return res


def _assert_rescale_needed(w, units):
    """Some checked row and wave group has a log2-sum of weights more than
    130 above the group's fixed reference: its row sum exceeds 2^130 relative
    to that reference, so at least one lane's partial sum passes 2^128 and
    overflows fp32 -- the unit's result is right only if the rescaling pass
    ran."""
    gaps = [g for g in _rescale_gaps(w, units) if g is not None]
    n_over = sum(g > 130 for g in gaps)
    log(f"  rows needing the rescale in {n_over} of {len(gaps)} checked units "
        f"(largest gap {max(gaps):.0f} log2 units)")
    assert n_over > 0


RESCALE = [
    # a large softmax scale on ordinary inputs: the global row maximum sits
    # far above the first tile's
    ("lut64_scale_16", dict(seed=320, B=1, H=2, S=2048, block=64,
                            density=0.5, vbs_mode="partial"), 16.0, None),
    # one later key block scaled by 16 (exact in bf16)
    ("lut64_planted_block", dict(seed=321, B=1, H=2, S=2048, block=64,
                                 density=0.5, vbs_mode="partial"), 0.5, 24),
    ("lut64_planted_tiny", dict(seed=322, B=1, H=2, S=4096, block=64,
                                density=0.8, vbs_mode="tiny"), 0.5, 56),
    ("bitmap128_planted_block", dict(seed=323, B=1, H=2, S=2048, block=128,
                                     form="bitmap", density=0.5,
                                     vbs_mode="edges"), 0.5, 11),
    ("lut128_planted_block", dict(seed=324, B=2, H=2, S=2048, block=128,
                                  count_mode="uniform", vbs_mode="partial"),
     0.5, 9),
    # more units than a split launch takes: one wave group per unit
    ("wide_lut64_scale_16", dict(seed=326, B=1, H=36, S=1024, block=64,
                                 density=0.5, vbs_mode="partial"), 16.0, None),
    ("wide_bitmap64_planted_block", dict(seed=327, B=2, H=18, S=1024,
                                         block=64, form="bitmap", density=0.5,
                                         vbs_mode="edges"), 0.5, 11),
    # fp8: the block's K scale times 16
    ("fp8_lut64_planted_scale", dict(seed=325, B=1, H=2, S=2048, block=64,
                                     kv="fp8", density=0.5,
                                     vbs_mode="partial"), 0.5, 20),
]


@pytest.mark.parametrize("label,kw,scale,plant", RESCALE,
                         ids=[c[0] for c in RESCALE])
def test_rescaling_pass_parity(label, kw, scale, plant):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    w.sm_scale = scale
    if plant is not None:
        rows = slice(plant * w.block, (plant + 1) * w.block)
        if w.kv_fp8:
            ks = w.k_scale.clone()
            ks[:, :, plant] *= 16.0
            w.k_scale = ks
        else:
            k = w.k.clone()
            k[:, :, rows] = k[:, :, rows] * 16  # power of two: exact in bf16
            w.k = k
    log(f"[softmax] rescale {label} sm_scale={scale} planted={plant}")
    units = _units(w) or list(range(w.n_units))
    _parity(w, label)
    _assert_rescale_needed(w, units)
