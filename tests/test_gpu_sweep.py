"""Seeded random sweep of the forward and backward passes over the space of
shapes and options: batch, query and K/V heads, query and key lengths,
block size, selection form, count and valid-count modes, density, shared
metadata, K/V type.  Every drawn case is compared with the oracle at the
LSE tolerance of the parity cases (1e-3) and the O bound derived from the
bf16 roundings (see test_forward_sweep)."""

import random

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from tests.gpu_helpers import (check, log, run_gpu, run_oracle,
                               scaled_input_bounds, to_dev)
from tests.test_gpu_bwd import check_grads, dout_of, gpu_bwd, oracle_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


VBS = ("full", "random", "partial", "zero_some", "edges", "tiny")
# K/V types of the 24 forward cases: half bf16, a quarter fp8, the rest codebook
KV = ("bf16", "fp8", "bf16", "i8cb", "bf16", "fp8", "bf16", "i4cb") * 3


def draw(seed: int, backward: bool):
    r = random.Random(seed)
    block = r.choice((64, 128))
    Hk = r.choice((1, 2))
    H = Hk * r.choice((1, 2, 3))
    NQ = r.randint(1, 6)
    NK = r.randint(1, 24)
    kw = dict(B=r.choice((1, 2)), H=H, Hk=Hk, S=NQ * block, Sk=NK * block,
              block=block, form=r.choice(("lut", "bitmap")),
              density=r.choice((0.1, 0.3, 0.6, 1.0)),
              vbs_mode=r.choice(VBS), shared_meta=r.random() < 0.2)
    if kw["form"] == "lut":
        kw["count_mode"] = r.choice(("fixed", "uniform"))
        kw["sort"] = r.random() < 0.5
    if not backward:
        kw["kv"] = KV[(seed - 1000) % len(KV)]
    return kw


def _gpu_forward(w):
    """run_gpu, with the codebooks passed for codebook-coded K/V."""
    if not w.kv_codebook:
        return run_gpu(w)
    d = to_dev(w)
    kw = dict(block=w.block, sm_scale=w.sm_scale, k_scale=d["k_scale"],
              v_scale=d["v_scale"], k_codebook=w.k_codebook.cuda(),
              v_codebook=w.v_codebook.cuda())
    if w.form == "lut":
        out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"],
                                   d["q2k_num"], d["vbs"],
                                   meta_strides=w.meta_strides, **kw)
    else:
        out, lse = bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                                      mask_strides=w.mask_strides, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", range(24))
def test_forward_sweep(case):
    kw = draw(1000 + case, backward=False)
    w = workloads.make_random(2000 + case, **kw)
    log(f"[sweep fwd {case}] {kw}")
    out, lse = _gpu_forward(w)
    o_ref, l_ref = run_oracle(w)
    o_gpu, l_gpu = out.float().cpu().numpy(), lse.cpu().numpy()
    # The drawn cases include rows that attend a handful of keys, whose O is
    # close to a single V row (|O| up to ~4 for N(0, 1) values, where bf16's
    # spacing is 2^-6): the bound derived from the roundings applies
    # (O to bf16: 2^-8 |O| with margin; P to bf16: 2^-9 max|V|).
    if w.kv_codebook:
        vmax = float(w.v_codebook.abs().max() * w.v_scale.max())
    elif w.kv_fp8:
        vmax = float((w.v.float() * w.v_scale.repeat_interleave(w.block, -1)
                      .unsqueeze(-1)).abs().max())
    else:
        vmax = float(w.v.float().abs().max())
    o_abs, o_rel = scaled_input_bounds(vmax)
    check(o_gpu, l_gpu, o_ref, l_ref, f"sweep{case}", o_rel=o_rel, o_abs=o_abs)


def draw_wide(seed: int):
    """A block-64 bf16 case with more work units than a key-split launch
    takes (BSA_FWD_KEY_SPLIT_MAX_UNITS), so one wave group sweeps each
    unit: the small sweep above runs split launches at block 64."""
    r = random.Random(seed)
    Hk = r.choice((1, 2, 4))
    NQ = r.randint(2, 6)
    B = r.choice((1, 2))
    lo = bsa.BSA_FWD_KEY_SPLIT_MAX_UNITS + 1
    g = -(-lo // (B * NQ * Hk))  # heads per K/V head that pass the threshold
    H = Hk * (g + r.randint(0, 2))
    NK = r.randint(1, 24)
    kw = dict(B=B, H=H, Hk=Hk, S=NQ * 64, Sk=NK * 64, block=64,
              form=r.choice(("lut", "bitmap")),
              density=r.choice((0.1, 0.3, 0.6, 1.0)),
              vbs_mode=r.choice(VBS), shared_meta=r.random() < 0.2)
    if kw["form"] == "lut":
        kw["count_mode"] = r.choice(("fixed", "uniform"))
        kw["sort"] = r.random() < 0.5
    return kw


@pytest.mark.parametrize("case", range(8))
def test_forward_sweep_wide(case):
    kw = draw_wide(6000 + case)
    w = workloads.make_random(7000 + case, **kw)
    assert w.n_units > bsa.BSA_FWD_KEY_SPLIT_MAX_UNITS
    log(f"[sweep fwd wide {case}] units={w.n_units} {kw}")
    out, lse = run_gpu(w)
    o_ref, l_ref = run_oracle(w)
    o_gpu, l_gpu = out.float().cpu().numpy(), lse.cpu().numpy()
    o_abs, o_rel = scaled_input_bounds(float(w.v.float().abs().max()))
    check(o_gpu, l_gpu, o_ref.reshape(o_gpu.shape), l_ref.reshape(l_gpu.shape),
          f"sweep_wide{case}", o_rel=o_rel, o_abs=o_abs)


@pytest.mark.parametrize("case", range(12))
def test_backward_sweep(case):
    kw = draw(3000 + case, backward=True)
    w = workloads.make_random(4000 + case, **kw)
    log(f"[sweep bwd {case}] {kw}")
    dout = dout_of(w, 5000 + case)
    check_grads(gpu_bwd(w, dout), oracle_bwd(w, dout), f"sweep_bwd{case}")
