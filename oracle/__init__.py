"""CPU oracle for block-sparse attention (forward and its gradients) -- TEST
INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code.  See ``bsa_oracle.h`` for the definition it computes and its citations.
"""

from .oracle import (  # noqa: F401
    KV_BF16,
    KV_FP8E4M3,
    KV_I4_CODEBOOK,
    KV_I8_CODEBOOK,
    LSE_EMPTY,
    bf16_value,
    build,
    bwd,
    codebook_index,
    fp8e4m3_value,
    fwd_bitmap,
    fwd_lut,
    key_counts,
    lib_path,
    mask_to_lut,
    num_threads,
)
