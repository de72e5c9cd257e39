"""The allocation-free backward entry point (bsa_bwd_lut_noalloc, called
through the C ABI) against bsa_bwd_lut with a caller-owned workspace, on two
calls in a row, the second with a smaller input.  Both run the same kernels
in the same order on the same inputs, so the gradients must be bitwise
equal."""

import ctypes

import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from block_sparse_attention_tile_amd import _lib
from tests.gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _noalloc_raw(w, d, out, dout, lse):
    """bsa_bwd_lut_noalloc through the raw C symbol; outputs pre-filled with
    NaN so an unwritten element shows up."""
    dq = torch.full_like(d["q"], float("nan"))
    dk = torch.full_like(d["k"], float("nan"))
    dv = torch.full_like(d["v"], float("nan"))
    sb, sh = w.meta_strides
    idx = d["q2k_idx"].to(torch.int32).contiguous()
    num = d["q2k_num"].to(torch.int32).contiguous()
    vbs = None if d["vbs"] is None else d["vbs"].to(torch.int32).contiguous()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = _lib.load().bsa_bwd_lut_noalloc(
        _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(out), _p(dout), _p(lse), _p(idx),
        _p(num), int(idx.shape[-1]), int(sb), int(sh), _p(vbs), float(w.sm_scale),
        _p(dq), _p(dk), _p(dv), w.B, w.H, w.Hk, w.S, w.Sk, w.D, w.block, st)
    assert rc == bsa.BSA_OK, bsa.bsa_status_str(rc)
    return dq, dk, dv


CASES = [
    ("larger", dict(seed=401, B=2, H=4, Hk=2, S=2048, Sk=2048, block=64,
                    count_mode="uniform", vbs_mode="partial")),
    ("smaller", dict(seed=402, B=1, H=2, S=512, block=64, density=0.5,
                     vbs_mode="random")),
]


def test_noalloc_backward_equals_workspace_backward_twice():
    for label, kw in CASES:
        kw = dict(kw)
        w = workloads.make_random(kw.pop("seed"), **kw)
        need = _lib.load().bsa_bwd_workspace_size(w.B, w.H, w.S, w.Sk, w.block)
        log(f"[noalloc] {label}: B{w.B} H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk} "
            f"blk{w.block} workspace {need} B")
        assert need <= bsa.BSA_NOALLOC_SCRATCH_BYTES
        d = to_dev(w)
        out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"],
                                   d["q2k_num"], d["vbs"], block=w.block,
                                   sm_scale=w.sm_scale,
                                   meta_strides=w.meta_strides)
        g = torch.Generator().manual_seed(7)
        dout = torch.randn(tuple(w.q.shape), generator=g).to(torch.bfloat16).cuda()
        ref = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse, block=w.block,
                          q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"],
                          variable_block_sizes=d["vbs"], sm_scale=w.sm_scale,
                          meta_strides=w.meta_strides)
        got = _noalloc_raw(w, d, out, dout, lse)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
                f"{label}: {name} differs from the workspace call"
        log(f"  {label}: dq, dk, dv bitwise equal")


def test_noalloc_binding_matches_raw_call():
    w = workloads.make_random(403, B=1, H=2, S=1024, block=128,
                              count_mode="uniform", vbs_mode="edges")
    d = to_dev(w)
    out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                               d["vbs"], block=w.block)
    dout = torch.ones_like(out)
    raw = _noalloc_raw(w, d, out, dout, lse)
    idx = d["q2k_idx"].to(torch.int32).contiguous()
    num = d["q2k_num"].to(torch.int32).contiguous()
    vbs = d["vbs"].to(torch.int32).contiguous()
    via = bsa.bsa_bwd_lut_noalloc(d["q"], d["k"], d["v"], out, dout, lse, idx, num,
                                  vbs, block=w.block)
    torch.cuda.synchronize()
    for a, b in zip(raw, via):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
