"""The two routes of fp8 K/V give the same bits: widened inside the
attention kernel (``fp8_route="kernel"``), or widened to bf16 in a pass of
their own (the codebook dequantisation with the 256 fp8 values as levels)
and then loaded by the scaled-bf16 kernel (``"widen"``, the default past
one launch of units).  Both decode every code exactly and fold the
per-block scales in the same places, over the same per-block tiles."""

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


def _run(w, d, route):
    kw = dict(block=w.block, sm_scale=w.sm_scale, k_scale=d["k_scale"],
              v_scale=d["v_scale"], fp8_route=route)
    if w.form == "lut":
        return bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                               d["vbs"], meta_strides=w.meta_strides, **kw)
    return bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                              mask_strides=w.mask_strides, **kw)


CASES = [
    ("lut64_gqa_rect", dict(seed=941, B=1, H=4, Hk=2, S=2048, Sk=4096, block=64,
                            kv="fp8", density=0.4, vbs_mode="partial")),
    ("lut128_edges", dict(seed=942, B=2, H=3, S=1024, block=128, kv="fp8",
                          count_mode="uniform", vbs_mode="edges")),
    ("bitmap64_tiny", dict(seed=943, B=1, H=2, S=512, block=64, kv="fp8",
                           form="bitmap", density=0.7, vbs_mode="tiny")),
    ("bitmap128_zero", dict(seed=944, B=1, H=2, S=1024, block=128, kv="fp8",
                            form="bitmap", density=0.5, vbs_mode="zero_some")),
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_fp8_routes_bitwise_equal(label, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    d = to_dev(w)
    log(f"[fp8 route] {label}: {w.n_units} units")
    o1, l1 = _run(w, d, "kernel")
    o2, l2 = _run(w, d, "widen")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), label
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), label


def test_fp8_routes_bitwise_equal_full_size():
    """The fp8 workload at full size (6 144 units, so "auto" widens first),
    in the benchmark's launch order."""
    w = workloads.make_config(4)
    assert w.kv_fp8 and bsa.api._widen_fp8(w.B, w.H, w.NQ, "auto")
    d = to_dev(w)
    log(f"[fp8 route] {w.name}: {w.n_units} units")
    order = bsa.bsa_unit_order_lut(d["q2k_idx"], d["q2k_num"], d["vbs"], B=w.B, H=w.H,
                                   S=w.S, Sk=w.Sk, block=w.block,
                                   meta_strides=w.meta_strides)
    outs = []
    for route in ("kernel", "auto"):
        outs.append(bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                                    d["vbs"], block=w.block, sm_scale=w.sm_scale,
                                    k_scale=d["k_scale"], v_scale=d["v_scale"],
                                    meta_strides=w.meta_strides, balance=False,
                                    qblock_order=order, fp8_route=route))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
