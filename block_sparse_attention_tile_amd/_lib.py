"""ctypes loader for the HIP library ``libbsa.so`` (built in-tree by
``block_sparse_attention_tile_amd.build``).  There is no fallback: if the
library is missing or does not load, every call raises."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

# The exported C symbols, as declared in include/bsa.h.
EXPORTS = ("bsa_fwd_lut", "bsa_fwd_lut_ordered", "bsa_unit_order_lut",
           "bsa_fwd_bitmap", "bsa_fwd_bitmap_ordered", "bsa_unit_order_bitmap",
           "bsa_mask_to_lut",
           "bsa_bwd_workspace_size", "bsa_bwd_lut", "bsa_bwd_bitmap",
           "bsa_bwd_lut_noalloc",
           "bsa_codebook_dequant", "bsa_status_str")

_lib = None


def load():
    """Loads (once) and returns the ctypes handle of libbsa.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_sparse_attention_tile_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.bsa_fwd_lut.restype = ctypes.c_int32
    lib.bsa_fwd_lut.argtypes = [
        P, P, P, i32, P, P, P, P, i32, i64, i64, P, f32, P, P,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_fwd_lut_ordered.restype = ctypes.c_int32
    lib.bsa_fwd_lut_ordered.argtypes = [
        P, P, P, i32, P, P, P, P, i32, i64, i64, P, P, f32, P, P,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_unit_order_lut.restype = ctypes.c_int32
    lib.bsa_unit_order_lut.argtypes = [
        P, P, i32, i64, i64, P, P, i32, i32, i32, i32, i32, P]
    lib.bsa_fwd_bitmap.restype = ctypes.c_int32
    lib.bsa_fwd_bitmap.argtypes = [
        P, P, P, i32, P, P, P, i64, i64, P, f32, P, P,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_fwd_bitmap_ordered.restype = ctypes.c_int32
    lib.bsa_fwd_bitmap_ordered.argtypes = [
        P, P, P, i32, P, P, P, i64, i64, P, P, f32, P, P,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_unit_order_bitmap.restype = ctypes.c_int32
    lib.bsa_unit_order_bitmap.argtypes = [
        P, i64, i64, P, P, i32, i32, i32, i32, i32, P]
    lib.bsa_mask_to_lut.restype = ctypes.c_int32
    lib.bsa_mask_to_lut.argtypes = [P, i64, i32, P, P, P]
    sz = ctypes.c_size_t
    lib.bsa_bwd_workspace_size.restype = sz
    lib.bsa_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.bsa_bwd_lut.restype = ctypes.c_int32
    lib.bsa_bwd_lut.argtypes = [
        P, P, P, P, P, P, P, P, i32, i64, i64, P, f32, P, P, P, P, sz,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_bwd_bitmap.restype = ctypes.c_int32
    lib.bsa_bwd_bitmap.argtypes = [
        P, P, P, P, P, P, P, i64, i64, P, f32, P, P, P, P, sz,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_bwd_lut_noalloc.restype = ctypes.c_int32
    lib.bsa_bwd_lut_noalloc.argtypes = [
        P, P, P, P, P, P, P, P, i32, i64, i64, P, f32, P, P, P,
        i32, i32, i32, i32, i32, i32, i32, P]
    lib.bsa_codebook_dequant.restype = ctypes.c_int32
    lib.bsa_codebook_dequant.argtypes = [P, i32, P, P, i64, P]
    lib.bsa_status_str.restype = ctypes.c_char_p
    lib.bsa_status_str.argtypes = [i32]
    _lib = lib
    return lib
