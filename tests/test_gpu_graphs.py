"""HIP graph capture of the library's calls.

The forward pass (LUT form in a key-split launch and in an ordered launch
of more units than run at once, bitmap form, fp8 K/V widened by the
binding), the backward pass with a
caller-owned workspace and the allocation-free backward are each captured
once into a torch CUDA graph (a hipGraph on ROCm) and replayed several
times, with eager library work, output resets and synchronisations between
the replays.  Every replay must reproduce the eager call's bits.  The
library records no memset (its scratch buffers are cleared by a fill
kernel) and allocates nothing; outputs, orders and workspaces are made
before the capture, except the backward binding's gradient tensors, which
torch places in the graph's pool."""

import ctypes

import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import workloads
from block_sparse_attention_tile_amd import _lib
from tests.gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits_equal(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _eager_noise(d):
    """Unrelated eager work between replays (a library call on other
    buffers and a device-wide reduction), then a synchronisation."""
    x = torch.randn(1 << 20, device="cuda")
    _ = (x * 2).sum().item()
    torch.cuda.synchronize()


def _replay_and_check(graph, outputs, refs, label, d):
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs, refs)):
            assert _bits_equal(a, b), f"{label}: replay {r}, output {i} differs"
        _eager_noise(d)
    log(f"  {label}: {REPLAYS} replays bit-identical to the eager call")


FWD = [
    # 128 units: the key-split launch
    ("lut64_key_split", dict(seed=501, B=2, H=4, S=1024, block=64,
                             count_mode="uniform", vbs_mode="partial"), False),
    # 1 280 units with a precomputed launch order
    ("lut64_ordered", dict(seed=502, B=1, H=20, S=4096, block=64, density=0.3,
                           vbs_mode="edges"), True),
    ("bitmap128", dict(seed=503, B=1, H=6, S=2048, block=128, form="bitmap",
                       density=0.4, vbs_mode="partial"), False),
    # fp8 K/V past one launch of units: the binding widens them to bf16
    # (a pass and a torch allocation inside the captured call)
    ("fp8_widened", dict(seed=504, B=1, H=20, S=4096, block=64, kv="fp8",
                         density=0.3, vbs_mode="partial"), True),
]


@pytest.mark.parametrize("label,kw,ordered", FWD, ids=[c[0] for c in FWD])
def test_forward_graph_replays_match_eager(label, kw, ordered):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    d = to_dev(w)
    log(f"[graph] forward {label}: {w.n_units} units")
    order = None
    if ordered:
        assert bsa.api.launch_order_pays(w.B, w.H, w.NQ)
        order = bsa.bsa_unit_order_lut(d["q2k_idx"], d["q2k_num"], d["vbs"],
                                       B=w.B, H=w.H, S=w.S, Sk=w.Sk,
                                       block=w.block,
                                       meta_strides=w.meta_strides)

    def call(out, lse):
        sc = dict(k_scale=d["k_scale"], v_scale=d["v_scale"])
        if w.form == "lut":
            bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"], d["q2k_num"],
                            d["vbs"], block=w.block, sm_scale=w.sm_scale,
                            meta_strides=w.meta_strides, out=out, lse=lse,
                            balance=False, qblock_order=order, **sc)
        else:
            bsa.bsa_fwd_bitmap(d["q"], d["k"], d["v"], d["mask"], d["vbs"],
                               block=w.block, sm_scale=w.sm_scale,
                               mask_strides=w.mask_strides, out=out, lse=lse,
                               balance=False, **sc)

    def buffers():
        return (torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda"),
                torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda"))

    ref_o, ref_l = buffers()
    call(ref_o, ref_l)  # eager reference (also the warm-up before capture)
    torch.cuda.synchronize()
    out, lse = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, lse)
    torch.cuda.synchronize()
    _replay_and_check(graph, [out, lse], [ref_o, ref_l], label, d)


def _backward_case():
    w = workloads.make_random(511, B=1, H=4, Hk=2, S=1024, block=64,
                              count_mode="uniform", vbs_mode="partial")
    d = to_dev(w)
    out, lse = bsa.bsa_fwd_lut(d["q"], d["k"], d["v"], d["q2k_idx"],
                               d["q2k_num"], d["vbs"], block=w.block,
                               sm_scale=w.sm_scale, meta_strides=w.meta_strides)
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(tuple(w.q.shape), generator=g).to(torch.bfloat16).cuda()
    torch.cuda.synchronize()
    return w, d, out, lse, dout


def test_backward_graph_replays_match_eager():
    w, d, out, lse, dout = _backward_case()
    log(f"[graph] backward with a caller workspace: {w.n_units} units")
    need = int(_lib.load().bsa_bwd_workspace_size(w.B, w.H, w.S, w.Sk, w.block))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        return bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout, lse, block=w.block,
                           q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"],
                           variable_block_sizes=d["vbs"], sm_scale=w.sm_scale,
                           meta_strides=w.meta_strides, workspace=ws)

    refs = [t.clone() for t in call()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grads = call()
    torch.cuda.synchronize()
    _replay_and_check(graph, list(grads), refs, "backward", d)


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def test_noalloc_backward_graph_replays_match_eager():
    """The allocation-free entry point is for callers under graph capture:
    captured through the C ABI after one eager call (which looks up the
    library's scratch address on this device)."""
    w, d, out, lse, dout = _backward_case()
    log(f"[graph] allocation-free backward: {w.n_units} units")
    sb, sh = w.meta_strides
    vbs = d["vbs"]

    def call(dq, dk, dv):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = _lib.load().bsa_bwd_lut_noalloc(
            _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(out), _p(dout), _p(lse),
            _p(d["q2k_idx"]), _p(d["q2k_num"]), int(d["q2k_idx"].shape[-1]),
            int(sb), int(sh), _p(vbs), float(w.sm_scale), _p(dq), _p(dk), _p(dv),
            w.B, w.H, w.Hk, w.S, w.Sk, w.D, w.block, st)
        assert rc == bsa.BSA_OK, bsa.bsa_status_str(rc)

    def buffers():
        return (torch.empty_like(d["q"]), torch.empty_like(d["k"]),
                torch.empty_like(d["v"]))

    refs = buffers()
    call(*refs)
    torch.cuda.synchronize()
    grads = buffers()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(*grads)
    torch.cuda.synchronize()
    _replay_and_check(graph, list(grads), list(refs), "allocation-free backward", d)
