"""Calls on a side stream (``stream=``): every temporary the binding makes
(int32 copies of int64 metadata, dequantised codebook K/V, the backward
workspace) is made on the launch stream, and the results equal those of the
same calls on the current stream bitwise."""

import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from tests.gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _side_stream():
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    return s


def test_forward_backward_and_compaction_on_a_side_stream():
    w = workloads.make_random(301, B=1, H=2, S=512, block=64,
                              count_mode="uniform", vbs_mode="random")
    log("[streams] fwd/bwd/mask_to_lut on a side stream")
    d = to_dev(w)
    idx64, num64, vbs64 = (d["q2k_idx"].long(), d["q2k_num"].long(),
                           d["vbs"].long())
    g = torch.Generator().manual_seed(302)
    dout = torch.randn(tuple(w.q.shape), generator=g).to(torch.bfloat16).cuda()
    ref = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                          d["vbs"], block=64)
    ref_g = bsa.bsa_bwd(d["q"], d["k"], d["v"], ref[0], dout, ref[1], block=64,
                        q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"],
                        variable_block_sizes=d["vbs"])
    mask = (torch.rand((8, 8), generator=g) < 0.5).to(torch.int8).cuda()
    ref_m = bsa.bsa_mask_to_lut(mask)
    torch.cuda.synchronize()

    s = _side_stream()
    out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], idx64, num64, vbs64,
                               block=64, stream=s)
    grads = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse, block=64,
                        q2k_idx=idx64, q2k_num=num64, variable_block_sizes=vbs64,
                        stream=s)
    m = bsa.bsa_mask_to_lut(mask, stream=s)
    s.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    for a, b in zip(grads, ref_g):
        assert torch.equal(a, b)
    assert torch.equal(m[0], ref_m[0]) and torch.equal(m[1], ref_m[1])


def test_codebook_forward_on_a_side_stream():
    w = workloads.make_random(303, B=1, H=2, S=512, block=64, density=0.5,
                              kv="i4cb", vbs_mode="partial")
    log("[streams] codebook forward on a side stream")
    d = to_dev(w)
    kc, vc = w.k_codebook.cuda(), w.v_codebook.cuda()
    kw = dict(block=64, k_scale=d["k_scale"], v_scale=d["v_scale"],
              k_codebook=kc, v_codebook=vc)
    ref = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                          d["vbs"], **kw)
    torch.cuda.synchronize()
    s = _side_stream()
    out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                               d["vbs"], stream=s, **kw)
    s.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
