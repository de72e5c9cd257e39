"""GPU parity of the backward pass (bsa_bwd_lut / bsa_bwd_bitmap through the
C ABI) against the oracle's fp64 gradients on the same seeded inputs.

The GPU path takes the forward pass's own O and LSE (as a training step
would), so its error is the forward's bf16 rounding of O (through delta)
plus the bf16 rounding of P and dS as MFMA operands and of the outputs.
Each of these is a relative 2^-9 per term; the bound checked per gradient
tensor is max|gpu - ref| <= 2^-6 * max|ref| (four roundings of 2^-9 with a
factor 2 for cancellation in dS), and the relative L2 error <= 2^-7."""

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import oracle
import workloads
from tests.gpu_helpers import log, run_gpu, to_dev

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -6
L2_REL = 2.0 ** -7


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dout_of(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.q.shape, generator=g).to(torch.bfloat16)


def gpu_bwd(w, dout):
    d = to_dev(w)
    out, lse = run_gpu(w, dev_inputs=d)
    kw = dict(block=w.block, variable_block_sizes=d["vbs"], sm_scale=w.sm_scale)
    if w.form == "lut":
        g = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout.cuda(), lse,
                        q2k_idx=d["q2k_idx"], q2k_num=d["q2k_num"],
                        meta_strides=w.meta_strides, **kw)
    else:
        g = bsa.bsa_bwd(d["q"], d["k"], d["v"], out, dout.cuda(), lse,
                        mask=d["mask"], meta_strides=w.mask_strides, **kw)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in g]


def oracle_bwd(w, dout):
    kw = dict(block=w.block, vbs=w.vbs, sm_scale=w.sm_scale)
    if w.form == "lut":
        return oracle.bwd(w.q, w.k, w.v, dout, q2k_idx=w.q2k_idx,
                          q2k_num=w.q2k_num, meta_strides=w.meta_strides, **kw)
    return oracle.bwd(w.q, w.k, w.v, dout, mask=w.mask,
                      meta_strides=w.mask_strides, **kw)


def check_grads(got, ref, label):
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(a).any(), f"{label} {name}: NaN"
        scale = float(np.abs(r).max())
        err = float(np.abs(a - r).max())
        l2 = float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-30))
        log(f"  {label} {name}: max|ref|={scale:.3e} max|err|={err:.3e} "
            f"rel_l2={l2:.3e}")
        if scale == 0.0:
            assert err == 0.0, f"{label} {name}: must be exactly 0"
            continue
        assert err <= MAX_REL * scale, f"{label} {name}: max err {err:.3e}"
        assert l2 <= L2_REL, f"{label} {name}: rel L2 {l2:.3e}"


CASES = [
    ("lut64_half", dict(seed=201, B=1, H=2, S=512, block=64, density=0.5)),
    ("lut64_vbs_zero_some", dict(seed=202, B=2, H=2, S=512, block=64,
                                 count_mode="uniform", vbs_mode="zero_some")),
    ("lut128_uniform", dict(seed=203, B=1, H=2, S=1024, block=128,
                            count_mode="uniform", vbs_mode="partial")),
    ("bitmap64", dict(seed=204, B=1, H=2, S=512, block=64, form="bitmap",
                      density=0.5, vbs_mode="random")),
    ("bitmap128_shared", dict(seed=205, B=2, H=2, S=1024, block=128,
                              form="bitmap", shared_meta=True, density=0.3)),
    ("gqa_rect_lut64", dict(seed=206, B=2, H=4, Hk=2, S=512, Sk=768, block=64,
                            count_mode="uniform", vbs_mode="random")),
    ("gqa_rect_bitmap128", dict(seed=207, B=1, H=6, Hk=1, S=512, Sk=1024,
                                block=128, form="bitmap", density=0.4,
                                vbs_mode="partial")),
    ("lut64_count_zero_some", dict(seed=208, B=1, H=3, S=256, block=64,
                                   count_mode="uniform", max_kv=2)),
    ("lut64_one_block", dict(seed=209, B=1, H=2, S=64, block=64, density=1.0,
                             vbs_mode="partial")),
    ("lut64_dense", dict(seed=210, B=1, H=2, S=512, block=64, density=1.0)),
    # valid counts around 16-row edges (blocks with at most half their keys
    # valid split their query rows over two waves) and runs of 1-4-key
    # blocks (dq tiles spanning many blocks)
    ("lut64_vbs_edges", dict(seed=211, B=1, H=2, S=1024, block=64,
                             density=0.6, vbs_mode="edges")),
    ("lut128_vbs_edges", dict(seed=212, B=1, H=2, S=2048, block=128,
                              count_mode="uniform", vbs_mode="edges")),
    ("gqa_bitmap64_vbs_tiny", dict(seed=213, B=1, H=4, Hk=2, S=512, Sk=2048,
                                   block=64, form="bitmap", density=0.8,
                                   vbs_mode="tiny")),
    ("lut64_many_tiny", dict(seed=214, B=1, H=1, S=1024, Sk=16384, block=64,
                             density=0.9, vbs_mode="tiny")),
]


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(label, kw):
    kw = dict(kw)
    w = workloads.make_random(kw.pop("seed"), **kw)
    log(f"[bwd] {label} B{w.B} H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk} blk{w.block} "
        f"form={w.form}")
    dout = dout_of(w, 7)
    got = gpu_bwd(w, dout)
    ref = oracle_bwd(w, dout)
    check_grads(got, ref, label)


def test_backward_longest_key_block_list():
    """Key block 0 selected by every query unit of its K/V head: the dK/dV
    workgroup's map row and unit list hold BSA_MAX_KEY_BLOCKS entries (the
    largest LDS footprint) and it walks 16384 query steps."""
    w = workloads.make_random(216, B=1, H=4, Hk=1, S=4096 * 64, Sk=64 * 64,
                              block=64, density=2 / 64, max_kv=2,
                              vbs_mode="tiny")
    w.q2k_idx[:, 0] = 0
    assert w.Hk and (w.H // w.Hk) * w.NQ == bsa.BSA_MAX_KEY_BLOCKS
    log(f"[bwd] longest list H{w.H} Hk{w.Hk} S{w.S} Sk{w.Sk}")
    dout = dout_of(w, 10)
    got = gpu_bwd(w, dout)
    ref = oracle_bwd(w, dout)
    check_grads(got, ref, "longest_list")


def test_backward_all_rows_empty_gives_zero_gradients():
    w = workloads.make_random(211, B=1, H=2, S=256, block=64, count_mode="zero")
    log("[bwd] all rows empty")
    got = gpu_bwd(w, dout_of(w, 8))
    for t in got:
        assert (t == 0).all()


def test_backward_is_deterministic():
    w = workloads.make_random(212, B=1, H=2, S=512, block=64,
                              count_mode="uniform", vbs_mode="random")
    dout = dout_of(w, 9)
    log("[bwd] determinism")
    a = gpu_bwd(w, dout)
    b = gpu_bwd(w, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_full_size_jenga():
    """The Jenga workload at full size (1 024 units, the bitmap form), every
    gradient element against the oracle."""
    w = workloads.make_config(1)
    log(f"[bwd] {w.name}: {w.n_units} units")
    dout = dout_of(w, 401)
    check_grads(gpu_bwd(w, dout), oracle_bwd(w, dout), w.name)


def _query_slice(w, h, qb0, qb1):
    """Query blocks [qb0, qb1) of head h of a one-batch LUT workload as a
    workload of its own (the whole key sequence of K/V head h kept): the dq
    rows of those blocks depend on nothing else, so they equal the full
    launch's (dk and dv do not: other query blocks add to them)."""
    sb, sh = w.meta_strides
    rows = h * sh + torch.arange(qb0, qb1)
    r0, r1 = qb0 * w.block, qb1 * w.block
    n = qb1 - qb0
    return workloads.Workload(
        name=f"{w.name}[head {h}, q-blocks {qb0}..{qb1 - 1}]", B=1, H=1,
        S=r1 - r0, D=w.D, block=w.block, form="lut",
        q=w.q[:, h:h + 1, r0:r1].contiguous(), k=w.k[:, h:h + 1].contiguous(),
        v=w.v[:, h:h + 1].contiguous(), q2k_idx=w.q2k_idx[rows].contiguous(),
        q2k_num=w.q2k_num[rows].contiguous(), meta_strides=(n, n),
        vbs=w.vbs, sm_scale=w.sm_scale)


def test_backward_full_size_video_dq():
    """The video workload at full size (18 432 units, the benchmark's launch
    with its dq and dk/dv launch orders): dq of the first 32 query blocks of
    the first head and of the last 32 of the last head, every element,
    against the oracle run on those query blocks alone (the oracle's
    backward runs one K/V head per thread, so a whole video head would take
    minutes; dk and dv are checked at full size on Jenga above)."""
    w = workloads.make_config(2)
    assert w.B == 1 and w.Hk == w.H and w.form == "lut"
    log(f"[bwd] {w.name}: {w.n_units} units")
    dout = dout_of(w, 402)
    dq = gpu_bwd(w, dout)[0]
    for h, qb0, qb1 in ((0, 0, 32), (w.H - 1, w.NQ - 32, w.NQ)):
        ws = _query_slice(w, h, qb0, qb1)
        r0, r1 = qb0 * w.block, qb1 * w.block
        ref = oracle_bwd(ws, dout[:, h:h + 1, r0:r1].contiguous())[0]
        check_grads([dq[:, h:h + 1, r0:r1]], [ref], ws.name)
