"""Bit-exact parity of the GPU block-map -> look-up-table compaction
(bsa_mask_to_lut) with the oracle's compaction, and of the from-mask route
with the bitmap form of the forward pass."""

import numpy as np
import pytest
import torch

import block_sparse_attention_tile_amd as bsa
import oracle
import workloads
from tests.gpu_helpers import log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def random_mask(seed, rows, nk, density, values="01"):
    g = torch.Generator().manual_seed(seed)
    sel = torch.rand((rows, nk), generator=g) < density
    if values == "01":
        return sel.to(torch.int8)
    # arbitrary nonzero bytes (negative ones included) mean "selected"
    v = torch.randint(-128, 128, (rows, nk), generator=g, dtype=torch.int32)
    v[v == 0] = 5
    return torch.where(sel, v, torch.zeros_like(v)).to(torch.int8)


def compare(mask_cpu, mask_dev=None, label=""):
    i_ref, n_ref = oracle.mask_to_lut(mask_cpu)
    m = mask_cpu.cuda() if mask_dev is None else mask_dev
    idx, num = bsa.bsa_mask_to_lut(m)
    torch.cuda.synchronize()
    assert np.array_equal(num.cpu().numpy(), n_ref.numpy()), f"{label}: num"
    assert np.array_equal(idx.cpu().numpy(), i_ref.numpy()), f"{label}: idx"


CASES = [
    # label, seed, rows, nk, density, values
    ("one_by_one", 1, 1, 1, 1.0, "01"),
    ("empty_rows", 2, 3, 5, 0.0, "01"),
    ("full_rows", 3, 4, 77, 1.0, "01"),
    ("ragged_63", 4, 7, 63, 0.5, "01"),
    ("exact_64", 5, 16, 64, 0.5, "bytes"),
    ("chunk_cross_257", 6, 5, 257, 0.3, "bytes"),
    ("chunk_exact_512", 7, 9, 512, 0.7, "01"),
    ("sparse_1000", 8, 33, 1000, 0.01, "01"),
    ("max_nk", 9, 2, 16384, 0.5, "bytes"),
    ("video_like", 10, 18432, 768, 96 / 768, "01"),
    # around the kernel's 1024-block passes (16 mask bytes per lane)
    ("pass_1023", 11, 6, 1023, 0.4, "bytes"),
    ("pass_1024", 12, 6, 1024, 0.6, "01"),
    ("pass_1025", 13, 6, 1025, 0.5, "bytes"),
    ("pass_2049_dense", 14, 3, 2049, 0.95, "01"),
    ("rows_4b_aligned_1000", 15, 9, 1000, 0.3, "bytes"),
]


@pytest.mark.parametrize("label,seed,rows,nk,density,values", CASES,
                         ids=[c[0] for c in CASES])
def test_mask_to_lut_bit_exact(label, seed, rows, nk, density, values):
    log(f"[mask_to_lut] {label} rows={rows} nk={nk} p={density}")
    compare(random_mask(seed, rows, nk, density, values), label=label)


def test_mask_to_lut_unaligned_rows_and_base():
    """Row starts that are not 4-byte aligned (odd nk, base offset 1) take
    the byte-wise path (4- and 16-byte aligned rows take word loads)."""
    m = random_mask(7, 40, 131, 0.4)
    big = torch.zeros(m.numel() + 1, dtype=torch.int8, device="cuda")
    big[1:] = m.reshape(-1).cuda()
    dev = big[1:].view(40, 131)
    assert dev.data_ptr() % 4 == 1
    log("[mask_to_lut] unaligned base")
    compare(m, mask_dev=dev, label="unaligned")


def test_mask_to_lut_leading_dims():
    """[B, H, NQ, NK] masks keep their shape: idx [B, H, NQ, NK], num
    [B, H, NQ]."""
    m = random_mask(8, 2 * 3 * 16, 16, 0.5).view(2, 3, 16, 16)
    idx, num = bsa.bsa_mask_to_lut(m.cuda())
    assert idx.shape == (2, 3, 16, 16) and num.shape == (2, 3, 16)
    i_ref, n_ref = oracle.mask_to_lut(m)
    assert torch.equal(idx.cpu(), i_ref) and torch.equal(num.cpu(), n_ref)


def test_mask_to_lut_empty_input():
    m = torch.zeros((0, 12), dtype=torch.int8, device="cuda")
    idx, num = bsa.bsa_mask_to_lut(m)
    assert idx.shape == (0, 12) and num.shape == (0,)


@pytest.mark.parametrize("cfg", [1, 3])
def test_from_mask_equals_bitmap_form(cfg):
    """The from-mask route (GPU compaction + LUT forward) and the bitmap form
    select the same key set, visited in the same ascending order: outputs
    are bitwise identical."""
    if cfg == 1:
        w = workloads.make_config(1)  # shared [64, 64] Jenga mask
        mask, strides = w.mask, w.mask_strides
    else:
        w = workloads.make_random(41, B=2, H=3, S=2048, block=128, form="bitmap",
                                  density=0.3, vbs_mode="random")
        mask, strides = w.mask, w.mask_strides
    log(f"[from_mask] {w.name} strides={strides}")
    d = to_dev(w)
    out_b, lse_b = run_gpu(w, dev_inputs=d)
    out_m, lse_m, idx, num = bsa.bsa_fwd_from_mask(
        d["q"], d["k"], d["v"], d["mask"], d["vbs"], block=w.block,
        sm_scale=w.sm_scale, mask_strides=strides)
    torch.cuda.synchronize()
    assert torch.equal(out_m.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(lse_m.view(torch.int32), lse_b.view(torch.int32))
    i_ref, n_ref = oracle.mask_to_lut(mask)
    assert torch.equal(idx.cpu(), i_ref) and torch.equal(num.cpu(), n_ref)
