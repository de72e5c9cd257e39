/*
 * bsa.h -- C ABI of the MI355X (gfx950) block-sparse attention forward.
 *
 * One work unit is the `block` query rows of query block qb of head h of
 * batch b.  It attends only to the keys of its selected key blocks, given
 * either as a per-row look-up table (`q2k_idx` with a per-row count
 * `q2k_num`, the VSA form of FastVideo "block_sparse_attn_sm100a.py") or as
 * an i8 bitmap `mask[q_block, k_block]` (the Jenga form of rocke
 * "sparse_attention.py", module docstring: nonzero = attend).  Keys at or
 * past a key block's `variable_block_sizes` entry are masked.  The pass
 * returns O and a per-row base-2 log-sum-exp (FastVideo
 * "block_sparse_attn_sm100a.py", module docstring: lse = max(qk*qk_scale) +
 * log2(l), [B, H, S] fp32):
 *
 *   t_j   = (q . k_j) * sm_scale * log2(e)          over attended keys j
 *   O     = sum_j 2^(t_j - m) v_j / sum_j 2^(t_j - m),   m = max_j t_j
 *   LSE   = m + log2(sum_j 2^(t_j - m))
 *
 * A row with no attended key gets O = +0 exactly and LSE = BSA_LSE_EMPTY
 * (`is_supported` docstring of the same page: count-0 rows give exactly-zero
 * output and a finite LSE sentinel).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers.  The caller allocates and owns
 *    every buffer and keeps it alive until the work on `stream` completes.
 *    The library allocates no device memory, keeps no state between calls
 *    and is re-entrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    The call only enqueues work; it never synchronises.
 *  - Validation is static only (shapes, pointers, alignment, finite
 *    sm_scale); no device
 *    memory is read on the host.  On any error the status is returned,
 *    nothing is launched and `out`/`lse` are left untouched.
 *  - Device-side metadata is not validated; out-of-range values have the
 *    defined behaviour listed with each argument (no out-of-bounds access).
 */
#ifndef BSA_H
#define BSA_H

#include <float.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* LSE of a query row that attends to no key: the lowest finite float, a
 * finite stand-in for log2(0) that carries weight 0 when partial results are
 * merged. */
#define BSA_LSE_EMPTY (-FLT_MAX)

/* Largest supported number of key blocks S/block (LDS holds one byte and
 * one 32-bit list entry per key block per work unit). */
#define BSA_MAX_KEY_BLOCKS 16384

/* Largest number of query blocks S/block per (batch, head) that
 * bsa_unit_order_lut sorts (LDS holds one 64-bit key per query block). */
#define BSA_MAX_ORDER_QBLOCKS 4096

/* Forward launches with block 64, bf16 K/V and at most this many work units
 * (B*H*S/block) split each unit's attended keys between two wave groups of
 * its workgroup and merge the two partial results (O, row maximum, row sum)
 * in a fixed order: so few units all run at once (two such workgroups per
 * compute unit on 256 CUs), and the longest unit sets the time.  The result
 * is deterministic for given sizes and metadata; it can differ in the last
 * bits from the same unit computed in a larger launch (the partial sums are
 * added in another order). */
#define BSA_FWD_KEY_SPLIT_MAX_UNITS 512

typedef enum {
  BSA_OK = 0,
  BSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  BSA_ERR_SHAPE = 2,       /* a size is <= 0, S or Sk not a multiple of block,
                              or H not a multiple of Hk                    */
  BSA_ERR_UNSUPPORTED = 3, /* valid but not built: D != 128, block not 64/128,
                              too many key blocks, unknown kv dtype           */
  BSA_ERR_ALIGN = 4,       /* q, k, v or out not 16-byte aligned              */
  BSA_ERR_HIP = 5,         /* the HIP launch reported an error                */
  BSA_ERR_VALUE = 6        /* a scalar argument outside its domain: sm_scale
                              not finite                                      */
} bsa_status;

typedef enum {
  BSA_KV_BF16 = 0,   /* K and V are bf16 [B, H, S, D]                          */
  BSA_KV_FP8E4M3 = 1, /* K and V are OCP fp8 e4m3 ("fn") bytes [B, H, S, D],
                        each key block dequantised as code value times its
                        fp32 scale (rocke "sage_attention.py", module
                        docstring: K/V dequantised per block before the score
                        and the PV product).  Widened inside the kernel.
                        Equivalent, bit for bit: bsa_codebook_dequant with
                        kind BSA_CODEBOOK_I8 on the same bytes and the 256
                        fp8 values as the table (entry l = the value of byte
                        l ^ 0x80), then BSA_KV_BF16_SCALED with the same
                        scales; faster on launches of many units, at the
                        cost of bf16 copies of K and V                        */
  BSA_KV_BF16_SCALED = 2 /* K and V are bf16 values [B, H, S, D] times their
                        per-block fp32 scale: the form the codebook modes of
                        the same page take after bsa_codebook_dequant (value
                        = codebook[code], scale applied here, exactly as for
                        fp8: folded into the score scale and into P)          */
} bsa_kv_dtype;

typedef enum {
  BSA_CODEBOOK_I8 = 0, /* int8 codes, 256-entry table at code + 128           */
  BSA_CODEBOOK_I4 = 1  /* two int4 codes per byte (element 2i in the low
                          nibble, two's complement), 16 entries at code + 8 */
} bsa_codebook_kind;

/*
 * bsa_fwd_lut -- VSA (look-up-table) form.
 *
 *  q            bf16 [B, H, S, D], contiguous (BHSD), 16-byte aligned.
 *  k, v         [B, Hk, Sk, D] contiguous, bf16 or fp8 e4m3 per kv_dtype,
 *               16-byte aligned.  Query head h reads K/V head h / (H/Hk)
 *               (grouped-query attention; Hk = H is ordinary attention).
 *  kv_dtype     a bsa_kv_dtype value.
 *  k_scale,     fp32 [B, Hk, Sk/block]: per-(b, K/V head, key block) scales;
 *  v_scale      required for BSA_KV_FP8E4M3, ignored (may be NULL) for bf16.
 *  q2k_idx      int32 rows x max_kv: selected key-block indices of a row.
 *               Only entries below the row's count are read.  Entries
 *               outside [0, Sk/block) are skipped; order and repetitions do
 *               not matter (the row is a set).
 *  q2k_num      int32 per row: the count, clamped to [0, max_kv].
 *  max_kv       row length of q2k_idx (>= 1).
 *  meta_stride_b, meta_stride_h
 *               the metadata row of unit (b, h, qb) is
 *               b*meta_stride_b + h*meta_stride_h + qb (in rows).
 *               (H*S/block, S/block) = one row per unit; (0, 0) = one
 *               [S/block, max_kv] table shared by every batch and head.
 *  variable_block_sizes
 *               int32 [Sk/block] shared by every batch and head: valid keys
 *               of each key block, clamped to [0, block]; keys at or past it
 *               are masked.  NULL = every block full.
 *  sm_scale     natural-log softmax scale (1/sqrt(D) is the usual value).
 *               Any finite value: zero gives every attended key the same
 *               weight, a negative value reverses the ranking.  NaN or
 *               +-inf returns BSA_ERR_VALUE.  Per-block K/V scales (fp8,
 *               scaled bf16) may likewise be zero or negative: a block's
 *               keys are code value times scale, exactly.
 *  out          bf16 [B, H, S, D] contiguous, 16-byte aligned; every element
 *               is written.
 *  lse          fp32 [B, H, S] base-2 LSE, or NULL to skip it.
 *  B, H, Hk     batch, query heads, key/value heads (H a multiple of Hk).
 *  S, Sk        query and key sequence lengths, multiples of block
 *               (rocke "sparse_attention.py" specs carry seqlen_q and
 *               seqlen_k and separate query / KV head counts).
 *  D            head dimension; must be 128.
 *  block        64 or 128: the query-block and key-block size.
 *  stream       hipStream_t (void*), NULL = null stream.
 */
bsa_status bsa_fwd_lut(const void* q, const void* k, const void* v,
                       int32_t kv_dtype, const float* k_scale,
                       const float* v_scale, const int32_t* q2k_idx,
                       const int32_t* q2k_num, int32_t max_kv,
                       int64_t meta_stride_b, int64_t meta_stride_h,
                       const int32_t* variable_block_sizes, float sm_scale,
                       void* out, float* lse, int32_t B, int32_t H, int32_t Hk,
                       int32_t S, int32_t Sk, int32_t D, int32_t block,
                       void* stream);

/*
 * bsa_unit_order_lut -- launch order of the LUT-form work units.  Not an
 * operation of the pages: a scheduling aid for the forward launch.  For
 * every (b, h) it writes the permutation of the S/block query blocks by
 * decreasing rank value, ties by increasing query block, so that
 * bsa_fwd_lut_ordered starts its heavy units first, finishes on light ones
 * and runs units of similar length and selection side by side.  Over unit
 * (b, h, qb)'s first clamp(q2k_num, 0, max_kv) entries inside
 * [0, Sk/block): count = the sum of the entries' valid keys
 * (variable_block_sizes clamped to [0, block]; repeated entries count
 * twice: an estimate, exact for rows without repetitions), mean = the
 * entries' block indices summed, times 1023, divided by (number of entries
 * * max(Sk/block - 1, 1)), truncated (0 without entries); rank value =
 * min(count / 64, 2^21 - 1) * 1024 + 1023 - mean (integer division).
 *
 *  q2k_idx, q2k_num, max_kv, meta_stride_b, meta_stride_h,
 *  variable_block_sizes, B, H, S, Sk, block
 *               exactly as for bsa_fwd_lut.
 *  order        int32 [B*H*(S/block)], device memory, written in full:
 *               entry (b*H + h)*(S/block) + i is the i-th query block of
 *               (b, h) in launch order.
 *  stream       hipStream_t (void*), NULL = null stream.
 *
 * Deterministic.  Errors: BSA_ERR_NULL, BSA_ERR_SHAPE (sizes, strides,
 * max_kv as for bsa_fwd_lut), BSA_ERR_UNSUPPORTED (block not 64/128,
 * S/block > BSA_MAX_ORDER_QBLOCKS, too many key blocks), BSA_ERR_HIP; on
 * error nothing is launched.
 */
bsa_status bsa_unit_order_lut(const int32_t* q2k_idx, const int32_t* q2k_num,
                              int32_t max_kv, int64_t meta_stride_b,
                              int64_t meta_stride_h,
                              const int32_t* variable_block_sizes,
                              int32_t* order, int32_t B, int32_t H, int32_t S,
                              int32_t Sk, int32_t block, void* stream);

/*
 * bsa_fwd_lut_ordered -- bsa_fwd_lut with the work units launched in a
 * given order.  Arguments as bsa_fwd_lut, plus:
 *
 *  qblock_order int32 [B*H*(S/block)], device memory: for every (b, h), a
 *               permutation of 0 .. S/block - 1 (bsa_unit_order_lut writes
 *               one); NULL = q-block order, i.e. bsa_fwd_lut.  Entries
 *               outside [0, S/block) are clamped into it; an order that is
 *               not a permutation leaves some query blocks unwritten.
 *
 * Every unit computes the same bits in any order, so the outputs equal
 * bsa_fwd_lut's exactly.
 */
bsa_status bsa_fwd_lut_ordered(const void* q, const void* k, const void* v,
                               int32_t kv_dtype, const float* k_scale,
                               const float* v_scale, const int32_t* q2k_idx,
                               const int32_t* q2k_num, int32_t max_kv,
                               int64_t meta_stride_b, int64_t meta_stride_h,
                               const int32_t* variable_block_sizes,
                               const int32_t* qblock_order, float sm_scale,
                               void* out, float* lse, int32_t B, int32_t H,
                               int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                               int32_t block, void* stream);

/*
 * bsa_fwd_bitmap -- Jenga (bitmap) form.  Arguments as bsa_fwd_lut, except:
 *
 *  mask         int8 rows x (Sk/block): nonzero = the key block is attended
 *               (rocke "sparse_attention.py", module docstring).
 *  mask_stride_b, mask_stride_h
 *               the mask row of unit (b, h, qb) is
 *               b*mask_stride_b + h*mask_stride_h + qb (in rows);
 *               (0, 0) = one [S/block, Sk/block] mask for every batch and
 *               head.
 */
bsa_status bsa_fwd_bitmap(const void* q, const void* k, const void* v,
                          int32_t kv_dtype, const float* k_scale,
                          const float* v_scale, const int8_t* mask,
                          int64_t mask_stride_b, int64_t mask_stride_h,
                          const int32_t* variable_block_sizes, float sm_scale,
                          void* out, float* lse, int32_t B, int32_t H,
                          int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                          int32_t block, void* stream);

/*
 * bsa_unit_order_bitmap -- launch order of the bitmap-form work units, as
 * bsa_unit_order_lut computes it for the LUT form (not an operation of the
 * pages: a scheduling aid).  Over the key blocks inside [0, Sk/block) that
 * unit (b, h, qb)'s mask row selects: count = the sum of their valid keys
 * (variable_block_sizes clamped to [0, block]; exact, a block is selected
 * once), mean and rank value as for bsa_unit_order_lut.
 *
 *  mask, mask_stride_b, mask_stride_h, variable_block_sizes, B, H, S, Sk,
 *  block        exactly as for bsa_fwd_bitmap.
 *  order        int32 [B*H*(S/block)], device memory, written in full (as
 *               for bsa_unit_order_lut).
 *  stream       hipStream_t (void*), NULL = null stream.
 *
 * Deterministic.  Errors: BSA_ERR_NULL, BSA_ERR_SHAPE (sizes, negative
 * strides), BSA_ERR_UNSUPPORTED (block not 64/128, S/block >
 * BSA_MAX_ORDER_QBLOCKS, too many key blocks), BSA_ERR_HIP; on error
 * nothing is launched.
 */
bsa_status bsa_unit_order_bitmap(const int8_t* mask, int64_t mask_stride_b,
                                 int64_t mask_stride_h,
                                 const int32_t* variable_block_sizes,
                                 int32_t* order, int32_t B, int32_t H, int32_t S,
                                 int32_t Sk, int32_t block, void* stream);

/*
 * bsa_fwd_bitmap_ordered -- bsa_fwd_bitmap with the work units launched in
 * a given order.  Arguments as bsa_fwd_bitmap, plus qblock_order as for
 * bsa_fwd_lut_ordered (NULL = q-block order, i.e. bsa_fwd_bitmap; entries
 * clamped into [0, S/block); not a permutation leaves query blocks
 * unwritten).  Every unit computes the same bits in any order, so the
 * outputs equal bsa_fwd_bitmap's exactly.
 */
bsa_status bsa_fwd_bitmap_ordered(const void* q, const void* k, const void* v,
                                  int32_t kv_dtype, const float* k_scale,
                                  const float* v_scale, const int8_t* mask,
                                  int64_t mask_stride_b, int64_t mask_stride_h,
                                  const int32_t* variable_block_sizes,
                                  const int32_t* qblock_order, float sm_scale,
                                  void* out, float* lse, int32_t B, int32_t H,
                                  int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                                  int32_t block, void* stream);

/*
 * bsa_mask_to_lut -- compaction of a block map into the look-up-table form
 * (the `map_to_index` step that FastVideo "block_sparse_attn_sm100a.py"
 * runs before its from-mask launch, `block_sparse_attn_sm100a_from_mask`).
 *
 *  mask         int8 [rows, nk] row-major, device memory: nonzero = the key
 *               block is selected.  No alignment required.
 *  rows         number of rows (>= 0; 0 launches nothing).
 *  nk           key blocks per row, 1 <= nk <= BSA_MAX_KEY_BLOCKS.
 *  q2k_idx      int32 [rows, nk], written in full: row r holds its selected
 *               key blocks in ascending order, then -1 up to nk.
 *  q2k_num      int32 [rows]: the number of selected key blocks of each row.
 *  stream       hipStream_t (void*), NULL = null stream.
 *
 * The result feeds bsa_fwd_lut with max_kv = nk and the mask's row strides,
 * and gives the same attention as bsa_fwd_bitmap on the mask.  Exact
 * (integer) result.  Errors: BSA_ERR_SHAPE (rows < 0 or nk <= 0),
 * BSA_ERR_UNSUPPORTED (nk too large), BSA_ERR_NULL, BSA_ERR_HIP; on error
 * nothing is launched.
 */
bsa_status bsa_mask_to_lut(const int8_t* mask, int64_t rows, int32_t nk,
                           int32_t* q2k_idx, int32_t* q2k_num, void* stream);

/*
 * Backward pass: gradients of sum(O * dout) with respect to q, k, v for the
 * forward pass with bf16 K/V (the LSE output exists for this pairing:
 * FastVideo "block_sparse_attn_sm100a.py" keeps the LSE-producing path for
 * forward/backward pairing).  With t = (q . k) * sm_scale * log2(e) over a
 * unit's attended keys:
 *
 *   P = 2^(t - LSE),  dP = dout V^T,  delta = rowsum(dout * out),
 *   dS = P * (dP - delta),
 *   dq = sm_scale * dS K,  dk = sm_scale * dS^T Q,  dv = P^T dout
 *
 * (the chain rule of softmax attention; K/V head h/(H/Hk) receives the
 * gradients of all its query heads).  Rows with no attended key give dq = 0;
 * keys past a block's valid count and blocks nobody selects give dk = dv = 0.
 *
 *  q, k, v, sizes, metadata, variable_block_sizes, sm_scale
 *               exactly as passed to the forward call (bf16 K/V only).
 *  out, lse     the forward call's outputs for these inputs (lse must not
 *               be NULL); 16-byte aligned.
 *  dout         bf16 [B, H, S, D], 16-byte aligned.
 *  dq           bf16 [B, H, S, D]; dk, dv bf16 [B, Hk, Sk, D]; 16-byte
 *               aligned; every element is written.
 *  workspace    device memory of at least bsa_bwd_workspace_size(...) bytes,
 *               256-byte aligned, owned by the caller, free for the library
 *               to overwrite during the call (it holds delta, the
 *               key-block -> query-block selection map and the launch
 *               orders of the dq units -- LUT form, as bsa_unit_order_lut
 *               computes it -- and of the dk/dv units: heaviest first, for
 *               launches of more than 1024 units).
 *               Calls that overlap on the same workspace race.
 *  workspace_bytes  its size; a smaller value is BSA_ERR_SHAPE.
 *
 * Errors as the forward calls (plus BSA_ERR_UNSUPPORTED when (H/Hk)*S/block
 * exceeds BSA_MAX_KEY_BLOCKS); on error nothing is launched.  The result is
 * deterministic: every gradient element is accumulated by one workgroup in a
 * fixed order (no atomics).
 */
size_t bsa_bwd_workspace_size(int32_t B, int32_t H, int32_t S, int32_t Sk,
                              int32_t block);

bsa_status bsa_bwd_lut(const void* q, const void* k, const void* v,
                       const void* out, const void* dout, const float* lse,
                       const int32_t* q2k_idx, const int32_t* q2k_num,
                       int32_t max_kv, int64_t meta_stride_b,
                       int64_t meta_stride_h,
                       const int32_t* variable_block_sizes, float sm_scale,
                       void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, int32_t B, int32_t H, int32_t Hk,
                       int32_t S, int32_t Sk, int32_t D, int32_t block,
                       void* stream);

bsa_status bsa_bwd_bitmap(const void* q, const void* k, const void* v,
                          const void* out, const void* dout, const float* lse,
                          const int8_t* mask, int64_t mask_stride_b,
                          int64_t mask_stride_h,
                          const int32_t* variable_block_sizes, float sm_scale,
                          void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, int32_t B, int32_t H,
                          int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                          int32_t block, void* stream);

/* Size of the library-owned workspace of bsa_bwd_lut_noalloc, per GPU. */
#define BSA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * bsa_bwd_lut_noalloc -- bsa_bwd_lut for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * bsa_bwd_lut, without workspace / workspace_bytes: the workspace is the
 * library's own device array of BSA_NOALLOC_SCRATCH_BYTES, one per GPU,
 * allocated when the library is loaded on that GPU and held until the
 * process ends.  The call allocates and frees nothing.
 *
 *  - Sizes whose bsa_bwd_workspace_size(B, H, S, Sk, block) exceeds
 *    BSA_NOALLOC_SCRATCH_BYTES return BSA_ERR_UNSUPPORTED (nothing is
 *    launched); use bsa_bwd_lut with a workspace of your own then.
 *  - All calls on one GPU share the array: calls whose stream work
 *    overlaps on the same GPU race, so serialise them (one stream, or
 *    events).  Nothing in the array needs clearing by the caller; each call
 *    writes what it reads.
 *  - The current device must be the GPU of the tensors and the stream.
 */
bsa_status bsa_bwd_lut_noalloc(const void* q, const void* k, const void* v,
                               const void* out, const void* dout, const float* lse,
                               const int32_t* q2k_idx, const int32_t* q2k_num,
                               int32_t max_kv, int64_t meta_stride_b,
                               int64_t meta_stride_h,
                               const int32_t* variable_block_sizes, float sm_scale,
                               void* dq, void* dk, void* dv, int32_t B, int32_t H,
                               int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                               int32_t block, void* stream);

/*
 * bsa_codebook_dequant -- codebook K/V codes to bf16 values (rocke
 * "sage_attention.py": K/V stored as i8 or i4 codes of an f32 codebook,
 * dequantised as codebook[code] times the per-block scale).  Writes
 * out[i] = bf16(codebook[level(i)]) (round to nearest even); the per-block
 * scale is applied by the forward call with kv_dtype BSA_KV_BF16_SCALED.
 *
 *  codes     device memory: n_values int8 codes (kind BSA_CODEBOOK_I8,
 *            16-byte aligned) or n_values/2 bytes of packed int4 codes
 *            (BSA_CODEBOOK_I4, 8-byte aligned).
 *  codebook  fp32 device table of 256 (i8) or 16 (i4) entries.
 *  out       bf16 device buffer of n_values elements, 16-byte aligned.
 *  n_values  number of values, a multiple of 16 (0 launches nothing).
 *  stream    hipStream_t (void*), NULL = null stream.
 *
 * Exact given the bf16 rounding of the table.  Errors: BSA_ERR_UNSUPPORTED
 * (unknown kind), BSA_ERR_SHAPE, BSA_ERR_NULL, BSA_ERR_ALIGN, BSA_ERR_HIP;
 * on error nothing is launched.
 */
bsa_status bsa_codebook_dequant(const void* codes, int32_t kind,
                                const float* codebook, void* out,
                                int64_t n_values, void* stream);

/* Static text of a status code (never NULL). */
const char* bsa_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
