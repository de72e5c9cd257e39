"""Thin Python binding of the C ABI in ``include/bsa.h``.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``libbsa.so``.  PyTorch supplies device memory and the stream:
``torch.cuda.current_stream()``, or the stream given as the keyword
``stream=`` (every entry point takes it; the whole call then runs under
``torch.cuda.stream(stream)``); outputs are allocated here with
``torch.empty`` when not passed in.  Integer metadata is cast to contiguous
int32 as the FastVideo wrapper does (``block_sparse_attn_sm100a``).
"""

from __future__ import annotations

import contextlib
import ctypes
import functools
from typing import Optional, Tuple

import torch

from . import _lib

BSA_OK = 0
BSA_ERR_NULL = 1
BSA_ERR_SHAPE = 2
BSA_ERR_UNSUPPORTED = 3
BSA_ERR_ALIGN = 4
BSA_ERR_HIP = 5
BSA_ERR_VALUE = 6
BSA_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
BSA_KV_BF16 = 0
BSA_KV_FP8E4M3 = 1
BSA_KV_BF16_SCALED = 2
BSA_CODEBOOK_I8 = 0
BSA_CODEBOOK_I4 = 1
LSE_EMPTY = -3.4028234663852886e38  # BSA_LSE_EMPTY = -FLT_MAX
BSA_MAX_KEY_BLOCKS = 16384
BSA_MAX_ORDER_QBLOCKS = 4096
# forward launches (block 64, bf16 K/V) of at most this many units split each
# unit's keys over two wave groups of its workgroup
BSA_FWD_KEY_SPLIT_MAX_UNITS = 512

# A launch of at most this many work units runs them all at once (256 CUs
# hold up to 4 workgroups each), so their launch order cannot matter.
ORDER_MIN_UNITS = 1024


def launch_order_pays(B: int, H: int, NQ: int) -> bool:
    """Whether the LUT-form forward computes a launch order by default:
    more units than run at once, and few enough query blocks to sort."""
    return B * H * NQ > ORDER_MIN_UNITS and NQ <= BSA_MAX_ORDER_QBLOCKS


class BsaError(RuntimeError):
    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(f"bsa status {status}: {bsa_status_str(status)}")


def bsa_status_str(status: int) -> str:
    return _lib.load().bsa_status_str(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_stream(fn):
    """Runs the whole call under ``torch.cuda.stream(stream)`` when a stream
    is given, so the temporaries it makes (int32 and contiguous copies,
    dequantised K/V, the workspace) are produced on, ordered before and
    owned by the stream the kernels are launched on."""
    @functools.wraps(fn)
    def wrapped(*args, stream: Optional[torch.cuda.Stream] = None, **kw):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, **kw)
    return wrapped


def _cur_stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_device(device: torch.device, **tensors) -> None:
    """Every tensor the kernels read or write must be GPU memory on the
    device of ``q``: the library dereferences the raw pointers on the GPU."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be a tensor on {device}, got {t.device}")


def _need_elems(name: str, t: Optional[torch.Tensor], n: int) -> None:
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements; the call reads {n}")


def _need_out(name: str, t: torch.Tensor, shape, dtype) -> None:
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{tuple(shape)}")


def _meta_rows(B: int, H: int, NQ: int, sb: int, sh: int) -> int:
    """Metadata rows the kernels address: row(b, h, qb) = b*sb + h*sh + qb."""
    return (B - 1) * max(sb, 0) + (H - 1) * max(sh, 0) + NQ


def _check_meta(q, k, block, sb, sh, *, idx=None, num=None, mask=None,
                vbs=None, k_scale=None, v_scale=None) -> None:
    """Device and size checks of the metadata against what the kernels read
    (the C ABI takes raw pointers and cannot see buffer sizes)."""
    B, H, S, _ = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    _need_device(q.device, q2k_idx=idx, q2k_num=num, mask=mask,
                 variable_block_sizes=vbs, k_scale=k_scale, v_scale=v_scale)
    if block not in (64, 128) or S % block or Sk % block:
        return  # the library rejects these shapes before any launch
    NQ, NK = S // block, Sk // block
    rows = _meta_rows(B, H, NQ, sb, sh)
    if idx is not None:
        width = int(idx.shape[-1]) if idx.dim() > 0 else 0
        if width > 0 and idx.numel() // width < rows:
            raise ValueError(f"q2k_idx has {idx.numel() // width} rows; the "
                             f"strides address {rows}")
        _need_elems("q2k_num", num, rows)
    if mask is not None:
        if mask.dim() < 1 or int(mask.shape[-1]) != NK:
            raise ValueError(f"mask rows must hold Sk/block = {NK} bytes")
        _need_elems("mask", mask, rows * NK)
    _need_elems("variable_block_sizes", vbs, NK)
    _need_elems("k_scale", k_scale, B * Hk * NK)
    _need_elems("v_scale", v_scale, B * Hk * NK)


def _kv_dtype(k: torch.Tensor, v: torch.Tensor) -> int:
    if k.dtype != v.dtype:
        raise TypeError("k and v must have the same dtype")
    if k.dtype == torch.bfloat16:
        return BSA_KV_BF16
    if k.dtype == torch.float8_e4m3fn:
        return BSA_KV_FP8E4M3
    if k.dtype in (torch.int8, torch.uint8):
        return BSA_KV_BF16_SCALED  # codebook codes, dequantised first
    raise TypeError(f"unsupported k/v dtype {k.dtype}")


@_on_stream
def bsa_codebook_dequant(codes: torch.Tensor, codebook: torch.Tensor
                         ) -> torch.Tensor:
    """bf16 codebook values of codebook-coded K or V: int8 codes
    ``[..., D]`` (256-entry codebook) or uint8 bytes of packed int4 codes
    ``[..., D/2]`` (16-entry codebook).  Returns bf16 ``[..., D]``; the
    per-block scale is not applied."""
    if codes.dtype == torch.int8:
        kind, shape = BSA_CODEBOOK_I8, tuple(codes.shape)
    elif codes.dtype == torch.uint8:
        kind, shape = BSA_CODEBOOK_I4, tuple(codes.shape[:-1]) + (2 * codes.shape[-1],)
    else:
        raise TypeError("codes must be int8 (i8) or uint8 (packed i4)")
    if not codes.is_cuda:
        raise ValueError(f"codes must be a GPU tensor, got {codes.device}")
    codes = codes.contiguous()
    cb = codebook.to(device=codes.device, dtype=torch.float32).contiguous()
    if cb.numel() != (256 if kind == BSA_CODEBOOK_I8 else 16):
        raise ValueError("codebook must have 256 (i8) or 16 (i4) entries")
    out = torch.empty(shape, dtype=torch.bfloat16, device=codes.device)
    n = out.numel()
    rc = _lib.load().bsa_codebook_dequant(_ptr(codes), kind, _ptr(cb), _ptr(out),
                                          n, _cur_stream(codes))
    if rc != BSA_OK:
        raise BsaError(rc)
    return out


FP8_ROUTES = ("auto", "kernel", "widen")
_FP8_LEVELS = {}


def _fp8_levels(device) -> torch.Tensor:
    """The 256 fp8 e4m3 values as an i8 codebook: level l holds the value of
    the code byte l ^ 0x80 (level = code + 128, the codebook convention).
    Every value is exact in f32 and in bf16."""
    key = str(device)
    if key not in _FP8_LEVELS:
        b = (torch.arange(256, dtype=torch.int32) ^ 0x80).to(torch.uint8)
        _FP8_LEVELS[key] = b.view(torch.float8_e4m3fn).to(torch.float32).to(device)
    return _FP8_LEVELS[key]


def _widen_fp8(B: int, H: int, NQ: int, route: str) -> bool:
    """Whether fp8 K/V are widened to bf16 in a pass of their own before the
    forward (then the kernel loads them like scaled bf16) instead of inside
    the kernel.  The two give the same bits; the pass pays on launches of
    more units than run at once, where each key block is gathered many
    times ("auto")."""
    if route not in FP8_ROUTES:
        raise ValueError(f"fp8_route must be one of {FP8_ROUTES}")
    if route == "auto":
        return B * H * NQ > ORDER_MIN_UNITS
    return route == "widen"


def _i32(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    return None if t is None else t.to(torch.int32).contiguous()


def _prepare(q, k, v, k_scale, v_scale, out, lse, need_lse, block,
             k_codebook=None, v_codebook=None, fp8_route="auto"):
    if q.dtype != torch.bfloat16 or q.dim() != 4:
        raise TypeError("q must be a 4-D bf16 [B, H, S, D] tensor")
    if not q.is_cuda:
        raise ValueError(f"q must be a GPU tensor, got {q.device}")
    _need_device(q.device, k=k, v=v, out=out, lse=lse)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if k.dtype in (torch.int8, torch.uint8):
        if k_codebook is None or v_codebook is None:
            raise ValueError("codebook-coded k/v need k_codebook and v_codebook")
        if k.dtype != v.dtype:
            raise TypeError("k and v must have the same dtype")
        k = bsa_codebook_dequant(k, k_codebook)
        v = bsa_codebook_dequant(v, v_codebook)
        kvd = BSA_KV_BF16_SCALED
    elif k.dtype == torch.float8_e4m3fn and v.dtype == k.dtype and \
            _widen_fp8(int(q.shape[0]), int(q.shape[1]),
                       int(q.shape[2]) // block if block > 0 else 0, fp8_route):
        levels = _fp8_levels(q.device)
        k = bsa_codebook_dequant(k.view(torch.int8), levels)
        v = bsa_codebook_dequant(v.view(torch.int8), levels)
        kvd = BSA_KV_BF16_SCALED
    else:
        kvd = None
    if k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] \
            or k.shape[3] != q.shape[3] or q.shape[1] % k.shape[1] != 0:
        raise ValueError("q must be [B, H, S, D] and k, v [B, Hk, Sk, D] with "
                         "H a multiple of Hk")
    if kvd is None:
        kvd = _kv_dtype(k, v)
    if kvd != BSA_KV_BF16:
        if k_scale is None or v_scale is None:
            raise ValueError("fp8 and codebook k/v need k_scale and v_scale")
        k_scale = k_scale.to(torch.float32).contiguous()
        v_scale = v_scale.to(torch.float32).contiguous()
    else:
        k_scale = v_scale = None
    B, H, S, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need_out("out", out, q.shape, torch.bfloat16)
    if need_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if not need_lse:
        lse = None
    if lse is not None:
        _need_out("lse", lse, (B, H, S), torch.float32)
    return q, k, v, kvd, k_scale, v_scale, out, lse


def _launch_order(q, qblock_order, balance, B, H, NQ):
    """The given order (checked), True if one should be computed, or None
    (q-block order)."""
    if qblock_order is not None:
        _need_device(q.device, qblock_order=qblock_order)
        if qblock_order.dtype != torch.int32 or not qblock_order.is_contiguous():
            raise TypeError("qblock_order must be a contiguous int32 tensor")
        _need_elems("qblock_order", qblock_order, B * H * NQ)
        return qblock_order
    if balance and launch_order_pays(B, H, NQ):
        return True
    return None


@_on_stream
def bsa_fwd_lut(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                q2k_idx: torch.Tensor, q2k_num: torch.Tensor,
                variable_block_sizes: Optional[torch.Tensor] = None, *,
                block: int, sm_scale: Optional[float] = None,
                k_scale: Optional[torch.Tensor] = None,
                v_scale: Optional[torch.Tensor] = None,
                meta_strides: Optional[Tuple[int, int]] = None,
                need_lse: bool = True, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None,
                k_codebook: Optional[torch.Tensor] = None,
                v_codebook: Optional[torch.Tensor] = None,
                balance: bool = True,
                qblock_order: Optional[torch.Tensor] = None,
                fp8_route: str = "auto"):
    """VSA form.  Returns ``(out, lse)`` (``lse`` is None if not needed).
    ``q`` is ``[B, H, S, D]``, ``k``/``v`` ``[B, Hk, Sk, D]`` (query head h
    reads K/V head h // (H // Hk)).  ``meta_strides=(sb, sh)``: the LUT row
    of (b, h, qb) is ``b*sb + h*sh + qb``; default one row per unit.
    ``balance``: launch each head's query blocks heaviest first (an order
    computed on the GPU by ``bsa_unit_order_lut``; the outputs are the same
    bits either way); skipped beyond BSA_MAX_ORDER_QBLOCKS query blocks and
    for launches of at most ORDER_MIN_UNITS units, which all run at once.
    ``qblock_order``: an order computed beforehand (int32 ``[B*H*NQ]``, as
    ``bsa_unit_order_lut`` returns it) to launch with instead.
    ``fp8_route`` (fp8 K/V): "kernel" widens the codes inside the attention
    kernel, "widen" in a pass of their own first (bf16 K/V of the call's
    own), "auto" the latter past ORDER_MIN_UNITS units; same bits."""
    q, k, v, kvd, ks, vs, out, lse = _prepare(q, k, v, k_scale, v_scale, out,
                                              lse, need_lse, block, k_codebook,
                                              v_codebook, fp8_route)
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    idx = _i32(q2k_idx)
    num = _i32(q2k_num)
    vbs = _i32(variable_block_sizes)
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    _check_meta(q, k, block, int(sb), int(sh), idx=idx, num=num, vbs=vbs,
                k_scale=ks, v_scale=vs)
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    order = _launch_order(q, qblock_order, balance, B, H, NQ)
    if order is True:
        order = torch.empty(B * H * NQ, dtype=torch.int32, device=q.device)
        rc = _lib.load().bsa_unit_order_lut(
            _ptr(idx), _ptr(num), int(idx.shape[-1]), int(sb), int(sh),
            _ptr(vbs), _ptr(order), B, H, S, Sk, int(block), _cur_stream(q))
        if rc != BSA_OK:
            raise BsaError(rc)
    rc = _lib.load().bsa_fwd_lut_ordered(
        _ptr(q), _ptr(k), _ptr(v), kvd, _ptr(ks), _ptr(vs), _ptr(idx),
        _ptr(num), int(idx.shape[-1]), int(sb), int(sh), _ptr(vbs),
        _ptr(order), float(sm_scale), _ptr(out), _ptr(lse), B, H, Hk, S, Sk,
        D, int(block), _cur_stream(q))
    if rc != BSA_OK:
        raise BsaError(rc)
    return out, lse


@_on_stream
def bsa_unit_order_lut(q2k_idx: torch.Tensor, q2k_num: torch.Tensor,
                       variable_block_sizes: Optional[torch.Tensor] = None, *,
                       B: int, H: int, S: int, Sk: int, block: int,
                       meta_strides: Optional[Tuple[int, int]] = None):
    """Launch order of the LUT-form units: int32 ``[B*H*NQ]``, for every
    (b, h) its query blocks by decreasing attended-key count (ties by
    q-block), computed on the GPU."""
    idx = _i32(q2k_idx)
    num = _i32(q2k_num)
    vbs = _i32(variable_block_sizes)
    if not idx.is_cuda:
        raise ValueError(f"q2k_idx must be a GPU tensor, got {idx.device}")
    _need_device(idx.device, q2k_num=num, variable_block_sizes=vbs)
    NQ = S // block
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    if block in (64, 128) and S % block == 0 and Sk % block == 0:
        rows = _meta_rows(B, H, NQ, int(sb), int(sh))
        width = int(idx.shape[-1]) if idx.dim() > 0 else 0
        if width > 0 and idx.numel() // width < rows:
            raise ValueError(f"q2k_idx has {idx.numel() // width} rows; the "
                             f"strides address {rows}")
        _need_elems("q2k_num", num, rows)
        _need_elems("variable_block_sizes", vbs, Sk // block)
    order = torch.empty(max(B * H * NQ, 0), dtype=torch.int32, device=idx.device)
    rc = _lib.load().bsa_unit_order_lut(
        _ptr(idx), _ptr(num), int(idx.shape[-1]), int(sb), int(sh), _ptr(vbs),
        _ptr(order), B, H, S, Sk, int(block), _cur_stream(idx))
    if rc != BSA_OK:
        raise BsaError(rc)
    return order


@_on_stream
def bsa_unit_order_bitmap(mask: torch.Tensor,
                          variable_block_sizes: Optional[torch.Tensor] = None, *,
                          B: int, H: int, S: int, Sk: int, block: int,
                          mask_strides: Optional[Tuple[int, int]] = None):
    """Launch order of the bitmap-form units: int32 ``[B*H*NQ]``, for every
    (b, h) its query blocks by decreasing attended-key count (ties by
    q-block), computed on the GPU."""
    if not mask.is_cuda:
        raise ValueError(f"mask must be a GPU tensor, got {mask.device}")
    m = mask.to(torch.int8).contiguous()
    vbs = _i32(variable_block_sizes)
    _need_device(m.device, variable_block_sizes=vbs)
    NQ = S // block
    sb, sh = mask_strides if mask_strides is not None else (H * NQ, NQ)
    if block in (64, 128) and S % block == 0 and Sk % block == 0:
        rows = _meta_rows(B, H, NQ, int(sb), int(sh))
        _need_elems("mask", m, rows * (Sk // block))
        _need_elems("variable_block_sizes", vbs, Sk // block)
    order = torch.empty(max(B * H * NQ, 0), dtype=torch.int32, device=m.device)
    rc = _lib.load().bsa_unit_order_bitmap(
        _ptr(m), int(sb), int(sh), _ptr(vbs), _ptr(order), B, H, S, Sk,
        int(block), _cur_stream(m))
    if rc != BSA_OK:
        raise BsaError(rc)
    return order


@_on_stream
def bsa_fwd_bitmap(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   mask: torch.Tensor,
                   variable_block_sizes: Optional[torch.Tensor] = None, *,
                   block: int, sm_scale: Optional[float] = None,
                   k_scale: Optional[torch.Tensor] = None,
                   v_scale: Optional[torch.Tensor] = None,
                   mask_strides: Optional[Tuple[int, int]] = None,
                   need_lse: bool = True, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None,
                   k_codebook: Optional[torch.Tensor] = None,
                   v_codebook: Optional[torch.Tensor] = None,
                   balance: bool = True,
                   qblock_order: Optional[torch.Tensor] = None,
                   fp8_route: str = "auto"):
    """Jenga form.  ``mask`` is an int8 (or bool) tensor of rows of S/block
    bytes; ``mask_strides=(sb, sh)`` as in the LUT form ((0, 0) = one
    [NQ, NK] mask shared by all batches and heads).  Shapes as in the LUT
    form.  ``balance``, ``qblock_order`` and ``fp8_route`` as in the LUT
    form, with the order from ``bsa_unit_order_bitmap``."""
    q, k, v, kvd, ks, vs, out, lse = _prepare(q, k, v, k_scale, v_scale, out,
                                              lse, need_lse, block, k_codebook,
                                              v_codebook, fp8_route)
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    m = mask.to(torch.int8).contiguous()
    vbs = _i32(variable_block_sizes)
    sb, sh = mask_strides if mask_strides is not None else (H * NQ, NQ)
    _check_meta(q, k, block, int(sb), int(sh), mask=m, vbs=vbs, k_scale=ks,
                v_scale=vs)
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    order = _launch_order(q, qblock_order, balance, B, H, NQ)
    if order is True:
        order = torch.empty(B * H * NQ, dtype=torch.int32, device=q.device)
        rc = _lib.load().bsa_unit_order_bitmap(
            _ptr(m), int(sb), int(sh), _ptr(vbs), _ptr(order), B, H, S, Sk,
            int(block), _cur_stream(q))
        if rc != BSA_OK:
            raise BsaError(rc)
    rc = _lib.load().bsa_fwd_bitmap_ordered(
        _ptr(q), _ptr(k), _ptr(v), kvd, _ptr(ks), _ptr(vs), _ptr(m),
        int(sb), int(sh), _ptr(vbs), _ptr(order), float(sm_scale), _ptr(out),
        _ptr(lse), B, H, Hk, S, Sk, D, int(block), _cur_stream(q))
    if rc != BSA_OK:
        raise BsaError(rc)
    return out, lse


@_on_stream
def bsa_mask_to_lut(mask: torch.Tensor):
    """Compacts a block map ``mask [..., NK]`` (nonzero = selected) on the
    GPU into ``(q2k_idx [..., NK] int32, q2k_num [...] int32)``: ascending
    selected key blocks, then -1 padding."""
    if not mask.is_cuda:
        raise ValueError(f"mask must be a GPU tensor, got {mask.device}")
    m = mask.to(torch.int8).contiguous()
    if m.dim() < 1:
        raise ValueError("mask must have a key-block dimension")
    nk = int(m.shape[-1])
    rows = m.numel() // nk if nk > 0 else 0
    idx = torch.empty(m.shape, dtype=torch.int32, device=m.device)
    num = torch.empty(m.shape[:-1], dtype=torch.int32, device=m.device)
    rc = _lib.load().bsa_mask_to_lut(_ptr(m), int(rows), nk, _ptr(idx),
                                     _ptr(num), _cur_stream(m))
    if rc != BSA_OK:
        raise BsaError(rc)
    return idx, num


@_on_stream
def bsa_fwd_from_mask(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      mask: torch.Tensor,
                      variable_block_sizes: Optional[torch.Tensor] = None, *,
                      block: int, mask_strides: Optional[Tuple[int, int]] = None,
                      **kw):
    """The from-mask route: compaction on the GPU, then the LUT form.  Gives
    the same result as ``bsa_fwd_bitmap`` on the same mask; also returns the
    look-up table for reuse.  Returns ``(out, lse, q2k_idx, q2k_num)``."""
    idx, num = bsa_mask_to_lut(mask)
    out, lse = bsa_fwd_lut(q, k, v, idx.reshape(-1, idx.shape[-1]),
                           num.reshape(-1), variable_block_sizes, block=block,
                           meta_strides=mask_strides, **kw)
    return out, lse, idx, num


@_on_stream
def bsa_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, *,
            block: int, q2k_idx: Optional[torch.Tensor] = None,
            q2k_num: Optional[torch.Tensor] = None,
            mask: Optional[torch.Tensor] = None,
            variable_block_sizes: Optional[torch.Tensor] = None,
            sm_scale: Optional[float] = None,
            meta_strides: Optional[Tuple[int, int]] = None,
            workspace: Optional[torch.Tensor] = None):
    """Gradients ``(dq, dk, dv)`` of ``sum(out * dout)`` for the forward pass
    that produced ``out`` and ``lse`` from the same inputs (bf16 K/V).  LUT
    form if ``q2k_idx`` is given, else bitmap form (``mask``);
    ``meta_strides`` addresses the metadata rows of either form.  The
    workspace (delta and the key-block -> query-block map) is allocated here
    unless given (uint8, at least ``bsa_bwd_workspace_size`` bytes)."""
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or \
            v.dtype != torch.bfloat16:
        raise TypeError("the backward pass takes bf16 q, k, v")
    if not q.is_cuda:
        raise ValueError(f"q must be a GPU tensor, got {q.device}")
    _need_device(q.device, k=k, v=v, out=out, dout=dout, lse=lse,
                 workspace=workspace)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or \
            k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3] or \
            q.shape[1] % k.shape[1] != 0:
        raise ValueError("q must be [B, H, S, D] and k, v [B, Hk, Sk, D] with "
                         "H a multiple of Hk")
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    out, dout = out.contiguous(), dout.to(torch.bfloat16).contiguous()
    lse = lse.to(torch.float32).contiguous()
    B, H, S, D = q.shape
    if tuple(out.shape) != tuple(q.shape) or out.dtype != torch.bfloat16 or \
            tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, S):
        raise ValueError("out and dout must be bf16 like q, lse [B, H, S]")
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    lib = _lib.load()
    need = int(lib.bsa_bwd_workspace_size(B, H, S, Sk, int(block)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    vbs = _i32(variable_block_sizes)
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    st = _cur_stream(q)
    common_tail = (float(sm_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                   int(workspace.numel()), B, H, Hk, S, Sk, D, int(block), st)
    if q2k_idx is not None:
        idx, num = _i32(q2k_idx), _i32(q2k_num)
        _check_meta(q, k, block, int(sb), int(sh), idx=idx, num=num, vbs=vbs)
        rc = lib.bsa_bwd_lut(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                             _ptr(lse), _ptr(idx), _ptr(num), int(idx.shape[-1]),
                             int(sb), int(sh), _ptr(vbs), *common_tail)
    else:
        if mask is None:
            raise ValueError("give q2k_idx and q2k_num, or mask")
        m = mask.to(torch.int8).contiguous()
        _check_meta(q, k, block, int(sb), int(sh), mask=m, vbs=vbs)
        rc = lib.bsa_bwd_bitmap(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                _ptr(lse), _ptr(m), int(sb), int(sh), _ptr(vbs),
                                *common_tail)
    if rc != BSA_OK:
        raise BsaError(rc)
    return dq, dk, dv


def bsa_bwd_lut_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                        q2k_idx: torch.Tensor, q2k_num: torch.Tensor,
                        variable_block_sizes: Optional[torch.Tensor] = None, *,
                        block: int, sm_scale: Optional[float] = None,
                        meta_strides: Optional[Tuple[int, int]] = None,
                        dq: Optional[torch.Tensor] = None,
                        dk: Optional[torch.Tensor] = None,
                        dv: Optional[torch.Tensor] = None):
    """LUT-form backward through ``bsa_bwd_lut_noalloc``: the library's own
    per-GPU scratch replaces the workspace, so the C call allocates nothing
    (pass ``dq``, ``dk``, ``dv`` to keep this call allocation-free; metadata
    must already be contiguous int32).  Sizes whose workspace exceeds
    ``BSA_NOALLOC_SCRATCH_BYTES`` raise ``BsaError(BSA_ERR_UNSUPPORTED)``.
    Calls that overlap on one GPU race on the shared scratch."""
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or \
            v.dtype != torch.bfloat16:
        raise TypeError("the backward pass takes bf16 q, k, v")
    if not q.is_cuda:
        raise ValueError(f"q must be a GPU tensor, got {q.device}")
    _need_device(q.device, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk,
                 dv=dv)
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    for name, t, shape, dt in (("q", q, (B, H, S, D), torch.bfloat16),
                               ("k", k, (B, Hk, Sk, D), torch.bfloat16),
                               ("v", v, (B, Hk, Sk, D), torch.bfloat16),
                               ("out", out, (B, H, S, D), torch.bfloat16),
                               ("dout", dout, (B, H, S, D), torch.bfloat16),
                               ("lse", lse, (B, H, S), torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of shape {shape}")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor like {ref.shape}")
    NQ = S // block
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    for name, t in (("q2k_idx", q2k_idx), ("q2k_num", q2k_num),
                    ("variable_block_sizes", variable_block_sizes)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    _check_meta(q, k, block, int(sb), int(sh), idx=q2k_idx, num=q2k_num,
                vbs=variable_block_sizes)
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    rc = _lib.load().bsa_bwd_lut_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(q2k_idx), _ptr(q2k_num), int(q2k_idx.shape[-1]), int(sb), int(sh),
        _ptr(variable_block_sizes), float(sm_scale), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, Hk, S, Sk, D, int(block), _cur_stream(q))
    if rc != BSA_OK:
        raise BsaError(rc)
    return dq, dk, dv
