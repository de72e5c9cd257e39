"""ctypes wrapper around the C oracle (``libbsa_oracle.so``).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``.  Inputs are CPU torch tensors; outputs
are float64 numpy arrays.  Work units are numbered ``u = (b*H + h)*NQ + qb``;
with ``units=None`` every unit is computed and the outputs have the shapes
``[B, H, S, D]`` and ``[B, H, S]``, otherwise ``[n, block, D]`` and
``[n, block]`` for the n requested units.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

KV_BF16 = 0
KV_FP8E4M3 = 1
KV_I8_CODEBOOK = 2  # int8 codes, 256-entry codebook at code + 128
KV_I4_CODEBOOK = 3  # uint8 bytes of two i4 codes (even element low nibble)
# Finite LSE sentinel of a query row that attends to no key: the lowest finite
# binary32 value (a stand-in for log(0) that merges with weight 0).
LSE_EMPTY = float(np.finfo(np.float32).min)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libbsa_oracle.so")


def build() -> None:
    """Compile the oracle with gcc (``oracle/build.sh``)."""
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path()):
            build()
        lib = ctypes.CDLL(lib_path())
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.bsa_oracle_bf16_value.restype = f64
        lib.bsa_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.bsa_oracle_fp8e4m3_value.restype = f64
        lib.bsa_oracle_fp8e4m3_value.argtypes = [ctypes.c_uint8]
        lib.bsa_oracle_fwd_lut.restype = ctypes.c_int
        lib.bsa_oracle_codebook_index.restype = ctypes.c_int
        lib.bsa_oracle_codebook_index.argtypes = [ctypes.c_int, P, i64]
        lib.bsa_oracle_fwd_lut.argtypes = [
            P, P, P, ctypes.c_int, P, P, P, P, P, P, i32, i64, i64, P, f64,
            i32, i32, i32, i32, i32, i32, i32, P, i64, P, P]
        lib.bsa_oracle_fwd_bitmap.restype = ctypes.c_int
        lib.bsa_oracle_fwd_bitmap.argtypes = [
            P, P, P, ctypes.c_int, P, P, P, P, P, i64, i64, P, f64,
            i32, i32, i32, i32, i32, i32, i32, P, i64, P, P]
        lib.bsa_oracle_key_counts.restype = ctypes.c_int
        lib.bsa_oracle_key_counts.argtypes = [
            ctypes.c_int, P, P, i32, i64, i64, P, i64, i64, P,
            i32, i32, i32, i32, i32, P, i64, P]
        lib.bsa_oracle_bwd.restype = ctypes.c_int
        lib.bsa_oracle_bwd.argtypes = [
            ctypes.c_int, P, P, P, P, P, P, i32, P, i64, i64, P, f64,
            i32, i32, i32, i32, i32, i32, i32, P, P, P]
        lib.bsa_oracle_mask_to_lut.restype = ctypes.c_int
        lib.bsa_oracle_mask_to_lut.argtypes = [P, i64, i32, P, P]
        lib.bsa_oracle_num_threads.restype = ctypes.c_int
        lib.bsa_oracle_num_threads.argtypes = []
        _LIB = lib
    return _LIB


def num_threads() -> int:
    return int(_lib().bsa_oracle_num_threads())


def bf16_value(bits: int) -> float:
    return float(_lib().bsa_oracle_bf16_value(int(bits) & 0xFFFF))


def fp8e4m3_value(byte: int) -> float:
    return float(_lib().bsa_oracle_fp8e4m3_value(int(byte) & 0xFF))


def _cpu(t: torch.Tensor) -> torch.Tensor:
    assert t.device.type == "cpu", "oracle inputs must be CPU tensors"
    return t.contiguous()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _kv_bits(t: torch.Tensor):
    t = _cpu(t)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16), KV_BF16
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8), KV_FP8E4M3
    if t.dtype == torch.int8:
        return t, KV_I8_CODEBOOK
    if t.dtype == torch.uint8:
        return t, KV_I4_CODEBOOK
    raise TypeError(f"unsupported K/V dtype {t.dtype}")


def codebook_index(kind: int, codes: torch.Tensor, elem: int) -> int:
    """The oracle's codebook index of one element (kind 2 = i8, 3 = i4)."""
    c = _cpu(codes)
    return int(_lib().bsa_oracle_codebook_index(int(kind), _ptr(c), int(elem)))


def _units_arg(units, total):
    if units is None:
        return None, total
    u = torch.as_tensor(units, dtype=torch.int64).contiguous()
    return u, int(u.numel())


def _outputs(units, n, B, H, S, D, block):
    if units is None:
        return np.empty((B, H, S, D)), np.empty((B, H, S))
    return np.empty((n, block, D)), np.empty((n, block))


def _common(q, k, v, k_scale, v_scale, k_codebook=None, v_codebook=None):
    q = _cpu(q)
    assert q.dtype == torch.bfloat16 and q.dim() == 4
    kb, kdt = _kv_bits(k)
    vb, vdt = _kv_bits(v)
    assert kdt == vdt, "K and V must share a dtype"
    width = q.shape[3] // 2 if kdt == KV_I4_CODEBOOK else q.shape[3]
    assert k.dim() == 4 and k.shape == v.shape and k.shape[0] == q.shape[0]
    assert k.shape[3] == width and q.shape[1] % k.shape[1] == 0
    if kdt != KV_BF16:
        k_scale = _cpu(k_scale.to(torch.float32))
        v_scale = _cpu(v_scale.to(torch.float32))
    else:
        k_scale = v_scale = None
    if kdt in (KV_I8_CODEBOOK, KV_I4_CODEBOOK):
        n = 256 if kdt == KV_I8_CODEBOOK else 16
        k_codebook = _cpu(k_codebook.to(torch.float32))
        v_codebook = _cpu(v_codebook.to(torch.float32))
        assert k_codebook.numel() == n and v_codebook.numel() == n
    else:
        k_codebook = v_codebook = None
    return (q.view(torch.int16), kb, vb, kdt, k_scale, v_scale, k_codebook,
            v_codebook)


def fwd_lut(q, k, v, q2k_idx, q2k_num, vbs=None, *, block, sm_scale=None,
            k_scale=None, v_scale=None, meta_strides=None, units=None,
            k_codebook=None, v_codebook=None):
    """Oracle forward, LUT form.  ``q2k_idx`` is ``[..., max_kv]`` int32 and
    ``q2k_num`` the matching per-row counts; ``meta_strides=(sb, sh)`` gives
    the row of (b, h, qb) as ``b*sb + h*sh + qb`` (default: one row per
    (b, h, qb), i.e. ``(H*NQ, NQ)``).  ``q`` is ``[B, H, Sq, D]``,
    ``k``/``v`` ``[B, Hk, Sk, D]`` with H a multiple of Hk."""
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    qb_, kb_, vb_, kdt, ks, vs, kc, vc = _common(q, k, v, k_scale, v_scale,
                                                 k_codebook, v_codebook)
    idx = _cpu(q2k_idx.to(torch.int32))
    num = _cpu(q2k_num.to(torch.int32))
    max_kv = int(idx.shape[-1])
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    vbs_t = None if vbs is None else _cpu(vbs.to(torch.int32))
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    u, n = _units_arg(units, B * H * NQ)
    out, lse = _outputs(units, n, B, H, S, D, block)
    rc = _lib().bsa_oracle_fwd_lut(
        _ptr(qb_), _ptr(kb_), _ptr(vb_), kdt, _ptr(ks), _ptr(vs), _ptr(kc),
        _ptr(vc), _ptr(idx), _ptr(num), max_kv, sb, sh, _ptr(vbs_t), float(sm_scale),
        B, H, Hk, S, Sk, D, block, _ptr(u), n,
        out.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"bsa_oracle_fwd_lut failed (rc={rc})")
    return out, lse


def fwd_bitmap(q, k, v, mask, vbs=None, *, block, sm_scale=None,
               k_scale=None, v_scale=None, mask_strides=None, units=None,
               k_codebook=None, v_codebook=None):
    """Oracle forward, bitmap form.  ``mask`` is i8 rows of NK bytes;
    ``mask_strides=(sb, sh)`` as for the LUT (``(0, 0)`` = one shared
    ``[NQ, NK]`` mask).  Shapes as for ``fwd_lut``."""
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    qb_, kb_, vb_, kdt, ks, vs, kc, vc = _common(q, k, v, k_scale, v_scale,
                                                 k_codebook, v_codebook)
    m = _cpu(mask.to(torch.int8))
    sb, sh = mask_strides if mask_strides is not None else (H * NQ, NQ)
    vbs_t = None if vbs is None else _cpu(vbs.to(torch.int32))
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    u, n = _units_arg(units, B * H * NQ)
    out, lse = _outputs(units, n, B, H, S, D, block)
    rc = _lib().bsa_oracle_fwd_bitmap(
        _ptr(qb_), _ptr(kb_), _ptr(vb_), kdt, _ptr(ks), _ptr(vs), _ptr(kc),
        _ptr(vc), _ptr(m), sb, sh, _ptr(vbs_t), float(sm_scale),
        B, H, Hk, S, Sk, D, block, _ptr(u), n,
        out.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"bsa_oracle_fwd_bitmap failed (rc={rc})")
    return out, lse


def key_counts(*, B, H, S, block, q2k_idx=None, q2k_num=None, mask=None,
               vbs=None, meta_strides=None, mask_strides=None, units=None,
               Sk=None):
    """Integer decode: ``[n_units, NK]`` int32 attended-key counts per key
    block (LUT form if ``q2k_idx`` is given, else bitmap form).  ``S`` is the
    query length, ``Sk`` the key length (default ``S``)."""
    Sk = S if Sk is None else Sk
    NQ, NK = S // block, Sk // block
    vbs_t = None if vbs is None else _cpu(vbs.to(torch.int32))
    u, n = _units_arg(units, B * H * NQ)
    counts = np.empty((n, NK), dtype=np.int32)
    lib = _lib()
    if q2k_idx is not None:
        idx = _cpu(q2k_idx.to(torch.int32))
        num = _cpu(q2k_num.to(torch.int32))
        sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
        rc = lib.bsa_oracle_key_counts(
            0, _ptr(idx), _ptr(num), int(idx.shape[-1]), sb, sh, None, 0, 0,
            _ptr(vbs_t), B, H, S, Sk, block, _ptr(u), n,
            counts.ctypes.data_as(ctypes.c_void_p))
    else:
        m = _cpu(mask.to(torch.int8))
        sb, sh = mask_strides if mask_strides is not None else (H * NQ, NQ)
        rc = lib.bsa_oracle_key_counts(
            1, None, None, 0, 0, 0, _ptr(m), sb, sh,
            _ptr(vbs_t), B, H, S, Sk, block, _ptr(u), n,
            counts.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"bsa_oracle_key_counts failed (rc={rc})")
    return counts


def bwd(q, k, v, dout, *, block, q2k_idx=None, q2k_num=None, mask=None,
        vbs=None, sm_scale=None, meta_strides=None):
    """Oracle backward (bf16 K/V): gradients ``(dq, dk, dv)`` of
    ``sum(O * dout)``, float64 numpy arrays shaped like q, k, v.  LUT form if
    ``q2k_idx`` is given, else bitmap form (``mask``); ``meta_strides``
    addresses the metadata rows of either form (default one row per
    unit)."""
    B, H, S, D = q.shape
    Hk, Sk = int(k.shape[1]), int(k.shape[2])
    NQ = S // block
    qb_, kb_, vb_, kdt, _, _, _, _ = _common(q, k, v, None, None)
    assert kdt == KV_BF16, "the backward pass takes bf16 K/V"
    do = _cpu(dout)
    assert do.dtype == torch.bfloat16 and tuple(do.shape) == tuple(q.shape)
    do = do.view(torch.int16)
    sb, sh = meta_strides if meta_strides is not None else (H * NQ, NQ)
    vbs_t = None if vbs is None else _cpu(vbs.to(torch.int32))
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    dq = np.empty((B, H, S, D))
    dk = np.empty((B, Hk, Sk, D))
    dv = np.empty((B, Hk, Sk, D))
    if q2k_idx is not None:
        idx = _cpu(q2k_idx.to(torch.int32))
        num = _cpu(q2k_num.to(torch.int32))
        form, max_kv, m = 0, int(idx.shape[-1]), None
    else:
        idx = num = None
        form, max_kv, m = 1, 0, _cpu(mask.to(torch.int8))
    rc = _lib().bsa_oracle_bwd(
        form, _ptr(qb_), _ptr(kb_), _ptr(vb_), _ptr(do), _ptr(idx), _ptr(num),
        max_kv, _ptr(m), sb, sh, _ptr(vbs_t), float(sm_scale),
        B, H, Hk, S, Sk, D, block,
        dq.ctypes.data_as(ctypes.c_void_p), dk.ctypes.data_as(ctypes.c_void_p),
        dv.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError(f"bsa_oracle_bwd failed (rc={rc})")
    return dq, dk, dv


def mask_to_lut(mask):
    """Compaction of an i8 ``[..., NK]`` bitmap into ``(idx [..., NK],
    num [...])`` with ascending indices and -1 padding."""
    m = _cpu(mask.to(torch.int8))
    NK = int(m.shape[-1])
    rows = m.numel() // NK
    idx = torch.empty(m.shape, dtype=torch.int32)
    num = torch.empty(m.shape[:-1], dtype=torch.int32)
    rc = _lib().bsa_oracle_mask_to_lut(_ptr(m), rows, NK, _ptr(idx), _ptr(num))
    if rc != 0:
        raise ValueError(f"bsa_oracle_mask_to_lut failed (rc={rc})")
    return idx, num
