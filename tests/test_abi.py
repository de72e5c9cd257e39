"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/bsa.h declares, and rejects invalid static arguments before any HIP
call (no compute is launched here)."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_tile_amd import _lib, api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_exactly_the_exported_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # dynamic symbol table, independent of ctypes
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define BSA_MAX_KEY_BLOCKS (\d+)", text).group(1)) == \
        api.BSA_MAX_KEY_BLOCKS
    assert int(re.search(r"#define BSA_MAX_ORDER_QBLOCKS (\d+)", text).group(1)) == \
        api.BSA_MAX_ORDER_QBLOCKS
    assert int(re.search(r"#define BSA_FWD_KEY_SPLIT_MAX_UNITS (\d+)", text).group(1)) == \
        api.BSA_FWD_KEY_SPLIT_MAX_UNITS
    for name in ("OK", "ERR_NULL", "ERR_SHAPE", "ERR_UNSUPPORTED", "ERR_ALIGN",
                 "ERR_HIP", "ERR_VALUE", "KV_BF16", "KV_FP8E4M3", "KV_BF16_SCALED",
                 "CODEBOOK_I8", "CODEBOOK_I4"):
        m = re.search(r"\bBSA_%s\s*=\s*(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(api, "BSA_" + name), name


def test_status_strings():
    for s in range(7):
        assert api.bsa_status_str(s) != "unknown status"
    assert api.bsa_status_str(99) == "unknown status"


# Fake, 16-byte aligned device addresses: validation fails before anything
# is dereferenced or launched.
A = 0x10000


def lut(**over):
    args = dict(q=A, k=A, v=A, kv=0, ks=None, vs=None, idx=A, num=A, max_kv=4,
                sb=8, sh=8, vbs=None, scale=0.1, out=A, lse=None, B=1, H=1,
                Hk=1, S=512, Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_fwd_lut(*args.values())


def lut_ordered(**over):
    args = dict(q=A, k=A, v=A, kv=0, ks=None, vs=None, idx=A, num=A, max_kv=4,
                sb=8, sh=8, vbs=None, order=None, scale=0.1, out=A, lse=None,
                B=1, H=1, Hk=1, S=512, Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_fwd_lut_ordered(*args.values())


def unit_order(**over):
    args = dict(idx=A, num=A, max_kv=4, sb=8, sh=8, vbs=None, order=A, B=1,
                H=1, S=512, Sk=512, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_unit_order_lut(*args.values())


def bitmap(**over):
    args = dict(q=A, k=A, v=A, kv=0, ks=None, vs=None, mask=A, sb=8, sh=8,
                vbs=None, scale=0.1, out=A, lse=None, B=1, H=1, Hk=1, S=512,
                Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_fwd_bitmap(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BSA_ERR_NULL),
    (dict(k=None), api.BSA_ERR_NULL),
    (dict(v=None), api.BSA_ERR_NULL),
    (dict(out=None), api.BSA_ERR_NULL),
    (dict(idx=None), api.BSA_ERR_NULL),
    (dict(num=None), api.BSA_ERR_NULL),
    (dict(kv=1), api.BSA_ERR_NULL),             # fp8 without scales
    (dict(kv=1, ks=A), api.BSA_ERR_NULL),
    (dict(B=0), api.BSA_ERR_SHAPE),
    (dict(H=-1), api.BSA_ERR_SHAPE),
    (dict(S=500), api.BSA_ERR_SHAPE),           # not a multiple of block
    (dict(Sk=500), api.BSA_ERR_SHAPE),
    (dict(Sk=0), api.BSA_ERR_SHAPE),
    (dict(H=6, Hk=4), api.BSA_ERR_SHAPE),       # H not a multiple of Hk
    (dict(Hk=0), api.BSA_ERR_SHAPE),
    (dict(max_kv=0), api.BSA_ERR_SHAPE),
    (dict(sb=-1), api.BSA_ERR_SHAPE),
    (dict(D=64), api.BSA_ERR_UNSUPPORTED),
    (dict(block=32, S=512), api.BSA_ERR_UNSUPPORTED),
    (dict(block=256, S=512), api.BSA_ERR_UNSUPPORTED),
    (dict(kv=7), api.BSA_ERR_UNSUPPORTED),
    (dict(S=64 * 16385, Sk=64 * 16385), api.BSA_ERR_UNSUPPORTED),
    (dict(Sk=64 * 16385), api.BSA_ERR_UNSUPPORTED),  # > BSA_MAX_KEY_BLOCKS
    (dict(q=A + 8), api.BSA_ERR_ALIGN),
    (dict(out=A + 2), api.BSA_ERR_ALIGN),
])
def test_lut_rejects_invalid_static_arguments(over, status):
    assert lut(**over) == status
    # the ordered entry point validates identically (order = NULL or not)
    assert lut_ordered(**over) == status
    assert lut_ordered(order=A, **over) == status


@pytest.mark.parametrize("over,status", [
    (dict(idx=None), api.BSA_ERR_NULL),
    (dict(num=None), api.BSA_ERR_NULL),
    (dict(order=None), api.BSA_ERR_NULL),
    (dict(B=0), api.BSA_ERR_SHAPE),
    (dict(H=0), api.BSA_ERR_SHAPE),
    (dict(S=500), api.BSA_ERR_SHAPE),
    (dict(Sk=96), api.BSA_ERR_SHAPE),
    (dict(max_kv=0), api.BSA_ERR_SHAPE),
    (dict(sh=-1), api.BSA_ERR_SHAPE),
    (dict(block=32), api.BSA_ERR_UNSUPPORTED),
    (dict(S=64 * (api.BSA_MAX_ORDER_QBLOCKS + 1)), api.BSA_ERR_UNSUPPORTED),
    (dict(Sk=64 * 16385), api.BSA_ERR_UNSUPPORTED),
])
def test_unit_order_rejects_invalid_static_arguments(over, status):
    assert unit_order(**over) == status


def bitmap_ordered(**over):
    args = dict(q=A, k=A, v=A, kv=0, ks=None, vs=None, mask=A, sb=8, sh=8,
                vbs=None, order=None, scale=0.1, out=A, lse=None, B=1, H=1,
                Hk=1, S=512, Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_fwd_bitmap_ordered(*args.values())


def unit_order_bitmap(**over):
    args = dict(mask=A, sb=8, sh=8, vbs=None, order=A, B=1, H=1, S=512,
                Sk=512, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_unit_order_bitmap(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(mask=None), api.BSA_ERR_NULL),
    (dict(order=None), api.BSA_ERR_NULL),
    (dict(B=0), api.BSA_ERR_SHAPE),
    (dict(S=500), api.BSA_ERR_SHAPE),
    (dict(Sk=96), api.BSA_ERR_SHAPE),
    (dict(sb=-1), api.BSA_ERR_SHAPE),
    (dict(block=32), api.BSA_ERR_UNSUPPORTED),
    (dict(S=64 * (api.BSA_MAX_ORDER_QBLOCKS + 1)), api.BSA_ERR_UNSUPPORTED),
    (dict(Sk=64 * 16385), api.BSA_ERR_UNSUPPORTED),
])
def test_unit_order_bitmap_rejects_invalid_static_arguments(over, status):
    assert unit_order_bitmap(**over) == status


@pytest.mark.parametrize("over,status", [
    (dict(mask=None), api.BSA_ERR_NULL),
    (dict(q=None), api.BSA_ERR_NULL),
    (dict(S=100), api.BSA_ERR_SHAPE),
    (dict(Sk=96), api.BSA_ERR_SHAPE),
    (dict(H=3, Hk=2), api.BSA_ERR_SHAPE),
    (dict(sh=-3), api.BSA_ERR_SHAPE),
    (dict(D=256), api.BSA_ERR_UNSUPPORTED),
    (dict(v=A + 4), api.BSA_ERR_ALIGN),
])
def test_bitmap_rejects_invalid_static_arguments(over, status):
    assert bitmap(**over) == status
    # the ordered entry point validates identically (order = NULL or not)
    assert bitmap_ordered(**over) == status
    assert bitmap_ordered(order=A, **over) == status


def test_python_binding_checks_dtypes_before_calling():
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.float32)
    with pytest.raises(TypeError):
        api.bsa_fwd_lut(q, q, q, torch.zeros((1, 1), dtype=torch.int32),
                        torch.zeros((1,), dtype=torch.int32), block=64)


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16)
    idx = torch.zeros((1, 1), dtype=torch.int32)
    num = torch.ones((1,), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        api.bsa_fwd_lut(q, q, q, idx, num, block=64)
    with pytest.raises(ValueError, match="GPU"):
        api.bsa_fwd_bitmap(q, q, q, idx.to(torch.int8), block=64)
    with pytest.raises(ValueError, match="GPU"):
        api.bsa_bwd(q, q, q, q, q, torch.zeros((1, 1, 64)), block=64,
                    q2k_idx=idx, q2k_num=num)
    with pytest.raises(ValueError, match="GPU"):
        api.bsa_mask_to_lut(idx.to(torch.int8))
    with pytest.raises(ValueError, match="GPU"):
        api.bsa_codebook_dequant(torch.zeros((16,), dtype=torch.int8),
                                 torch.zeros((256,)))


def mask_lut(**over):
    args = dict(mask=A, rows=4, nk=8, idx=A, num=A, stream=None)
    args.update(over)
    return _lib.load().bsa_mask_to_lut(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(mask=None), api.BSA_ERR_NULL),
    (dict(idx=None), api.BSA_ERR_NULL),
    (dict(num=None), api.BSA_ERR_NULL),
    (dict(rows=-1), api.BSA_ERR_SHAPE),
    (dict(nk=0), api.BSA_ERR_SHAPE),
    (dict(nk=16385), api.BSA_ERR_UNSUPPORTED),
    (dict(rows=0), api.BSA_OK),                       # empty: nothing launched
    (dict(rows=0, mask=None, idx=None, num=None), api.BSA_OK),
])
def test_mask_to_lut_rejects_invalid_static_arguments(over, status):
    assert mask_lut(**over) == status


def bwd_lut(**over):
    args = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, idx=A, num=A, max_kv=4,
                sb=8, sh=8, vbs=None, scale=0.1, dq=A, dk=A, dv=A, ws=A,
                ws_bytes=1 << 30, B=1, H=1, Hk=1, S=512, Sk=512, D=128,
                block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_bwd_lut(*args.values())


def bwd_bitmap(**over):
    args = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, mask=A, sb=8, sh=8,
                vbs=None, scale=0.1, dq=A, dk=A, dv=A, ws=A, ws_bytes=1 << 30,
                B=1, H=1, Hk=1, S=512, Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_bwd_bitmap(*args.values())


def test_bwd_workspace_size_covers_delta_map_and_order():
    lib = _lib.load()
    # delta: B*H*S floats, map: B*H*NQ*NK bytes, launch orders: B*H*NQ and
    # B*H*NK int32; each region 256-aligned
    up = lambda x: (x + 255) // 256 * 256
    assert lib.bsa_bwd_workspace_size(2, 3, 512, 1024, 64) == \
        up(up(up(2 * 3 * 512 * 4) + 2 * 3 * 8 * 16) + 2 * 3 * 8 * 4) + 2 * 3 * 16 * 4
    assert lib.bsa_bwd_workspace_size(0, 3, 512, 512, 64) == 0


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BSA_ERR_NULL),
    (dict(lse=None), api.BSA_ERR_NULL),
    (dict(dout=None), api.BSA_ERR_NULL),
    (dict(ws=None), api.BSA_ERR_NULL),
    (dict(dk=None), api.BSA_ERR_NULL),
    (dict(idx=None), api.BSA_ERR_NULL),
    (dict(S=500), api.BSA_ERR_SHAPE),
    (dict(H=3, Hk=2), api.BSA_ERR_SHAPE),
    (dict(max_kv=0), api.BSA_ERR_SHAPE),
    (dict(ws_bytes=100), api.BSA_ERR_SHAPE),       # workspace too small
    (dict(D=64), api.BSA_ERR_UNSUPPORTED),
    (dict(block=32), api.BSA_ERR_UNSUPPORTED),
    (dict(H=64, Hk=1, S=64 * 512), api.BSA_ERR_UNSUPPORTED),  # G*NQ too big
    (dict(ws=A + 16), api.BSA_ERR_ALIGN),         # workspace needs 256 B
    (dict(lse=A + 4), api.BSA_ERR_ALIGN),
    (dict(dq=A + 8), api.BSA_ERR_ALIGN),
])
def test_bwd_rejects_invalid_static_arguments(over, status):
    assert bwd_lut(**over) == status


@pytest.mark.parametrize("args,status", [
    ((A, 0, A, A, 15, None), api.BSA_ERR_SHAPE),      # not a multiple of 16
    ((A, 0, A, A, -16, None), api.BSA_ERR_SHAPE),
    ((A, 5, A, A, 16, None), api.BSA_ERR_UNSUPPORTED),
    ((None, 0, A, A, 16, None), api.BSA_ERR_NULL),
    ((A, 1, None, A, 16, None), api.BSA_ERR_NULL),
    ((A + 8, 0, A, A, 16, None), api.BSA_ERR_ALIGN),  # i8 codes need 16 B
    ((A, 0, A, A + 8, 16, None), api.BSA_ERR_ALIGN),
    ((None, 0, None, None, 0, None), api.BSA_OK),      # empty: no launch
])
def test_codebook_dequant_rejects_invalid_static_arguments(args, status):
    assert _lib.load().bsa_codebook_dequant(*args) == status


def test_lut_accepts_scaled_bf16_mode_only_with_scales():
    assert lut(kv=2) == api.BSA_ERR_NULL
    assert lut(kv=2, ks=A) == api.BSA_ERR_NULL


def test_launch_order_only_when_units_exceed_one_generation():
    # more units than the 256 CUs hold at once, and at most
    # BSA_MAX_ORDER_QBLOCKS query blocks per head
    assert not api.launch_order_pays(1, 16, 64)          # Jenga: 1024 units
    assert api.launch_order_pays(1, 24, 768)             # video: 18432 units
    assert api.launch_order_pays(1, 1, 1025)
    assert not api.launch_order_pays(1, 1, 1024)
    assert not api.launch_order_pays(1, 2, api.BSA_MAX_ORDER_QBLOCKS + 1)
    assert api.launch_order_pays(1, 2, api.BSA_MAX_ORDER_QBLOCKS)


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), -float("inf")])
def test_non_finite_softmax_scale_is_rejected_by_every_entry_point(scale):
    assert lut(scale=scale) == api.BSA_ERR_VALUE
    assert lut_ordered(scale=scale) == api.BSA_ERR_VALUE
    assert bitmap(scale=scale) == api.BSA_ERR_VALUE
    assert bwd_lut(scale=scale) == api.BSA_ERR_VALUE
    assert bwd_bitmap(scale=scale) == api.BSA_ERR_VALUE
    # zero and negative scales are valid values, rejected only for other
    # reasons (here: the null K pointer)
    for ok in (0.0, -0.5):
        assert lut(scale=ok, k=None) == api.BSA_ERR_NULL


def bwd_noalloc(**over):
    args = dict(q=A, k=A, v=A, out=A, dout=A, lse=A, idx=A, num=A, max_kv=4,
                sb=8, sh=8, vbs=None, scale=0.1, dq=A, dk=A, dv=A, B=1, H=1, Hk=1,
                S=512, Sk=512, D=128, block=64, stream=None)
    args.update(over)
    return _lib.load().bsa_bwd_lut_noalloc(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), api.BSA_ERR_NULL),
    (dict(idx=None), api.BSA_ERR_NULL),
    (dict(S=500), api.BSA_ERR_SHAPE),
    (dict(max_kv=0), api.BSA_ERR_SHAPE),
    (dict(D=64), api.BSA_ERR_UNSUPPORTED),
    (dict(dq=A + 8), api.BSA_ERR_ALIGN),
    (dict(scale=float("nan")), api.BSA_ERR_VALUE),
    # workspace beyond the library's scratch: delta 4*B*H*S bytes plus the
    # B*H*NQ*NK byte map exceed BSA_NOALLOC_SCRATCH_BYTES
    (dict(B=1, H=64, Hk=64, S=64 * 256, Sk=64 * 2048), api.BSA_ERR_UNSUPPORTED),
])
def test_noalloc_backward_rejects_invalid_static_arguments(over, status):
    assert bwd_noalloc(**over) == status


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define BSA_NOALLOC_SCRATCH_BYTES \((\d+) \* (\d+) \* (\d+)\)", text)
    assert m
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == \
        api.BSA_NOALLOC_SCRATCH_BYTES
    # the largest size the tests use stays inside it
    assert _lib.load().bsa_bwd_workspace_size(24, 1, 49152, 49152, 64) <= \
        api.BSA_NOALLOC_SCRATCH_BYTES
