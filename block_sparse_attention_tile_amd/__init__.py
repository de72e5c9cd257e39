"""MI355X (gfx950) block-sparse attention forward.

The compute runs in the HIP library ``libbsa.so`` (C ABI in
``include/bsa.h``); this package only marshals torch tensors into it.
"""

from .api import (  # noqa: F401
    BSA_ERR_ALIGN,
    BSA_ERR_HIP,
    BSA_ERR_NULL,
    BSA_ERR_SHAPE,
    BSA_ERR_UNSUPPORTED,
    BSA_ERR_VALUE,
    BSA_CODEBOOK_I4,
    BSA_CODEBOOK_I8,
    BSA_KV_BF16,
    BSA_KV_BF16_SCALED,
    BSA_KV_FP8E4M3,
    BSA_FWD_KEY_SPLIT_MAX_UNITS,
    BSA_MAX_KEY_BLOCKS,
    BSA_MAX_ORDER_QBLOCKS,
    BSA_NOALLOC_SCRATCH_BYTES,
    BSA_OK,
    LSE_EMPTY,
    BsaError,
    bsa_bwd,
    bsa_bwd_lut_noalloc,
    bsa_codebook_dequant,
    bsa_fwd_bitmap,
    bsa_fwd_from_mask,
    bsa_fwd_lut,
    bsa_mask_to_lut,
    bsa_status_str,
    bsa_unit_order_bitmap,
    bsa_unit_order_lut,
)
