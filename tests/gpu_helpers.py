"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle on the same seeded inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import block_sparse_attention_tile_amd as bsa
import oracle

# Target tolerances for bf16 inputs: O max-abs 1e-2, LSE (base 2) 1e-3.
O_TOL = 1e-2
LSE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w, dev="cuda"):
    d = {}
    for name in ("q", "k", "v", "k_scale", "v_scale", "q2k_idx", "q2k_num",
                 "mask", "vbs", "k_codebook", "v_codebook"):
        t = getattr(w, name)
        d[name] = None if t is None else t.to(dev)
    return d


def run_gpu(w, *, need_lse=True, dev_inputs=None, prefill=float("nan")):
    """HIP forward of workload w.  Outputs are pre-filled (NaN by default) so
    an element the kernel forgets to write shows up."""
    d = dev_inputs if dev_inputs is not None else to_dev(w)
    out = torch.full(tuple(w.q.shape), prefill, dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((w.B, w.H, w.S), prefill, dtype=torch.float32,
                     device="cuda") if need_lse else None
    if w.form == "lut":
        bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                        d["vbs"], block=w.block, sm_scale=w.sm_scale,
                        k_scale=d["k_scale"], v_scale=d["v_scale"],
                        meta_strides=w.meta_strides, need_lse=need_lse,
                        out=out, lse=lse, k_codebook=d.get("k_codebook"),
                        v_codebook=d.get("v_codebook"))
    else:
        bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                           block=w.block, sm_scale=w.sm_scale,
                           k_scale=d["k_scale"], v_scale=d["v_scale"],
                           mask_strides=w.mask_strides, need_lse=need_lse,
                           out=out, lse=lse, k_codebook=d.get("k_codebook"),
                           v_codebook=d.get("v_codebook"))
    torch.cuda.synchronize()
    return out, lse


def run_oracle(w, units=None):
    kw = dict(block=w.block, sm_scale=w.sm_scale, k_scale=w.k_scale,
              v_scale=w.v_scale, units=units,
              k_codebook=w.k_codebook, v_codebook=w.v_codebook)
    if w.form == "lut":
        return oracle.fwd_lut(w.q, w.k, w.v, w.q2k_idx, w.q2k_num, w.vbs,
                              meta_strides=w.meta_strides, **kw)
    return oracle.fwd_bitmap(w.q, w.k, w.v, w.mask, w.vbs,
                             mask_strides=w.mask_strides, **kw)


def gather_units(w, out, lse, units):
    """Slices [n, block, D] / [n, block] of the GPU outputs for units."""
    o = out.view(w.n_units, w.block, w.D)
    idx = torch.as_tensor(units, dtype=torch.int64, device=out.device)
    og = o.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    lg = None
    if lse is not None:
        lg = lse.view(w.n_units, w.block).index_select(0, idx).cpu().numpy()
        lg = lg.astype(np.float64)
    return og, lg


def scaled_input_bounds(v_max_abs: float):
    """(o_abs, o_rel) for inputs beyond N(0, 1).  The kernel rounds each
    probability to bf16 before the PV product (relative error <= 2^-9), which
    moves O by at most 2^-9 * max|v|, and rounds O to bf16 (at most 2^-8 |O|
    with margin); 1e-2 covers the remaining fp32 accumulation."""
    return O_TOL + 2.0 ** -9 * v_max_abs, 2.0 ** -8


def check(o_gpu, l_gpu, o_ref, l_ref, label="", o_rel=0.0, o_abs=O_TOL):
    """Asserts parity: no NaN, O within o_abs (+ o_rel*|O|), LSE within
    LSE_TOL, and empty rows bit-exact (+0 output, the finite sentinel).

    The defaults are the target bound (max-abs 1e-2).  For inputs scaled
    beyond N(0, 1) the bound is derived from the arithmetic (see
    scaled_input_bounds)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    assert not np.isnan(o_gpu).any(), f"{label}: unwritten/NaN output"
    empty = l_ref == oracle.LSE_EMPTY
    excess = np.abs(o_gpu - o_ref) - o_rel * np.abs(o_ref)
    err_o = float(excess.max()) if o_gpu.size else 0.0
    msg = f"{label}: max(|dO|-{o_rel:g}|O|)={err_o:.3e}"
    if l_gpu is not None:
        l_gpu = np.asarray(l_gpu, dtype=np.float64)
        assert not np.isnan(l_gpu).any(), f"{label}: unwritten/NaN lse"
        assert (l_gpu[empty] == oracle.LSE_EMPTY).all(), f"{label}: sentinel"
        ne = ~empty
        err_l = float(np.abs(l_gpu[ne] - l_ref[ne]).max()) if ne.any() else 0.0
        msg += f" max|dLSE|={err_l:.3e}"
        assert err_l <= LSE_TOL, msg
    if empty.any():
        oe = o_gpu[empty]
        assert (oe == 0).all() and not np.signbit(oe).any(), \
            f"{label}: empty rows not +0"
    assert err_o <= o_abs, msg
    log("  " + msg + f" empty_rows={int(empty.sum())}")
    return err_o
