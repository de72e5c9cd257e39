/*
 * bsa_oracle.h -- plain, slow CPU oracle for block-sparse attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library: only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (exact sparse softmax attention, in double precision):
 *
 *   For one work unit (b, h, qb) -- the `block` query rows of query block qb
 *   of head h of batch b -- the attended key set is
 *       A   = selected key blocks of the unit
 *             LUT form   : { idx[row, j] : 0 <= j < clamp(num[row],0,max_kv),
 *                                          0 <= idx[row, j] < NK }
 *             bitmap form: { kb : mask[row, kb] != 0 }
 *       Kat = { kb*block + t : kb in A, 0 <= t < clamp(vbs[kb], 0, block) }
 *   and for every query row r of the unit
 *       t_j  = (q_r . kd_j) * sm_scale * log2(e)
 *       m    = max_j t_j,  w_j = 2^(t_j - m),  l = sum_j w_j
 *       O_r  = sum_j w_j vd_j / l,     LSE_r = m + log2(l)     (base 2)
 *   with O_r = 0 and LSE_r = -FLT_MAX when Kat is empty.
 *   kd/vd are the decoded keys/values: bf16 -> real, or fp8 e4m3 (OCP "fn"
 *   encoding) -> real times the per-(b, h, key block) fp32 scale.
 *
 * Sources (cited by page title and section):
 *   - FastVideo "block_sparse_attn_sm100a.py": module docstring (returns
 *     (out, lse), lse = max(qk*qk_scale) + log2(l), [B,H,S] fp32, 64/128
 *     token blocks) and the `is_supported` docstring (per-row counts in
 *     [0,max_kv], count-0 rows give zeros and a finite LSE sentinel, padding
 *     past the count never read, keys at or past variable_block_sizes masked).
 *   - rocke "sparse_attention.py": module docstring (Jenga MaskBitmap,
 *     1 = attend; VSA BlockLut/BlockCount) and `_stage_vsa_bitmap_to_lds`
 *     (the LUT entries below the count scattered into a per-q-block bitmap,
 *     duplicates idempotent) -- hence A is a *set*.
 *   - rocke "sage_attention.py": module docstring (fp8 K/V dequantised as
 *     code value times the per-block scale before the score and PV).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   qk_scale = sm_scale*log2(e); the finite sentinel is -FLT_MAX; an empty
 *   row caused by vbs = 0 on every selected block is treated like count 0;
 *   out-of-range idx below the count is skipped, num and vbs are clamped.
 *   sm_scale may be any finite value (zero: equal weights; negative:
 *   reversed ranking), and so may the fp8 block scales (zero included: the
 *   block's keys or values are then exactly zero); a non-finite sm_scale is
 *   an invalid argument.
 *
 * Work units are numbered u = (b*H + h)*NQ + qb.  Outputs are compact: for
 * the i-th requested unit, out[i][r][d] (r < block, d < D) and lse[i][r].
 * Passing units = NULL means all B*H*NQ units in order, so the compact layout
 * equals the [B,H,S,D] / [B,H,S] layout.
 *
 * Return value: 0 on success, nonzero on an invalid argument (nothing is
 * written then).  The caller owns every buffer.
 */
#ifndef BSA_ORACLE_H
#define BSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_KV_BF16 = 0,        /* bf16 values                                  */
  ORACLE_KV_FP8E4M3 = 1,     /* fp8 e4m3fn code value times the block scale  */
  ORACLE_KV_I8_CODEBOOK = 2, /* 256-entry f32 codebook[i8 + 128] times scale */
  ORACLE_KV_I4_CODEBOOK = 3  /* 16-entry f32 codebook[i4 + 8] times scale,
                                two codes per byte, even element low nibble */
};

/* Codebook index (0..255 or 0..15) of element `elem` of a codebook-coded
 * tensor (kv_dtype 2 or 3). */
int bsa_oracle_codebook_index(int kv_dtype, const void* base, int64_t elem);

/* Value of one bf16 bit pattern (exact). */
double bsa_oracle_bf16_value(uint16_t bits);
/* Value of one OCP fp8 e4m3fn byte (exact; NaN for S.1111.111). */
double bsa_oracle_fp8e4m3_value(uint8_t byte);

/* q: bf16 bits [B,H,Sq,D]; k, v: [B,Hk,Sk,D] bf16 bits, fp8 bytes or i8
 * codes, or [B,Hk,Sk,D/2] packed i4 codes, per kv_dtype, with H a multiple
 * of Hk (query head h reads K/V head h/(H/Hk));
 * k_scale, v_scale: fp32 [B,Hk,Sk/block] (all but bf16, else ignored);
 * k_codebook, v_codebook: fp32 tables (codebook modes, else ignored);
 * q2k_idx: int32 rows x max_kv, q2k_num: int32 rows, with
 * row = b*meta_stride_b + h*meta_stride_h + qb (qb < Sq/block), entries
 * naming key blocks in [0, Sk/block);
 * vbs: int32 [Sk/block] or NULL (all blocks full). */
int bsa_oracle_fwd_lut(const uint16_t* q, const void* k, const void* v,
                       int kv_dtype, const float* k_scale, const float* v_scale,
                       const float* k_codebook, const float* v_codebook,
                       const int32_t* q2k_idx, const int32_t* q2k_num,
                       int32_t max_kv, int64_t meta_stride_b,
                       int64_t meta_stride_h, const int32_t* vbs,
                       double sm_scale, int32_t B, int32_t H, int32_t Hk,
                       int32_t Sq, int32_t Sk, int32_t D, int32_t block,
                       const int64_t* units, int64_t n_units, double* out,
                       double* lse);

/* As above, with the selected set given by an i8 bitmap:
 * mask row = b*mask_stride_b + h*mask_stride_h + qb, NK bytes per row,
 * nonzero = attend. */
int bsa_oracle_fwd_bitmap(const uint16_t* q, const void* k, const void* v,
                          int kv_dtype, const float* k_scale,
                          const float* v_scale, const float* k_codebook,
                          const float* v_codebook, const int8_t* mask,
                          int64_t mask_stride_b, int64_t mask_stride_h,
                          const int32_t* vbs, double sm_scale, int32_t B,
                          int32_t H, int32_t Hk, int32_t Sq, int32_t Sk,
                          int32_t D, int32_t block, const int64_t* units,
                          int64_t n_units, double* out, double* lse);

/* Integer decode only: counts[i][kb] = number of attended keys of key block
 * kb for the i-th requested unit (clamp(vbs[kb],0,block) if kb is selected,
 * else 0).  form 0 = LUT (q2k_idx/q2k_num/max_kv/meta strides used),
 * form 1 = bitmap (mask/mask strides used). */
int bsa_oracle_key_counts(int form, const int32_t* q2k_idx,
                          const int32_t* q2k_num, int32_t max_kv,
                          int64_t meta_stride_b, int64_t meta_stride_h,
                          const int8_t* mask, int64_t mask_stride_b,
                          int64_t mask_stride_h, const int32_t* vbs, int32_t B,
                          int32_t H, int32_t Sq, int32_t Sk, int32_t block,
                          const int64_t* units, int64_t n_units,
                          int32_t* counts);

/* Gradients (dq [B,H,Sq,D], dk and dv [B,Hk,Sk,D], fp64, overwritten) of
 * sum(O * dout) for the forward pass with bf16 K/V, by the plain chain rule
 * of softmax attention over each unit's attended keys.  form 0 = LUT
 * (q2k_idx/q2k_num/max_kv), form 1 = bitmap (mask); meta_stride_b/h give
 * the metadata row of (b, h, qb) for either form.  dout: bf16 bits
 * [B,H,Sq,D].  Query rows with no attended key get dq = 0. */
int bsa_oracle_bwd(int form, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const uint16_t* dout,
                   const int32_t* q2k_idx, const int32_t* q2k_num,
                   int32_t max_kv, const int8_t* mask, int64_t meta_stride_b,
                   int64_t meta_stride_h, const int32_t* vbs, double sm_scale,
                   int32_t B, int32_t H, int32_t Hk, int32_t Sq, int32_t Sk,
                   int32_t D, int32_t block, double* dq, double* dk,
                   double* dv);

/* Compaction of a bitmap into the LUT form: for each of `rows` rows of NK
 * bytes, idx[row][0..n) = ascending positions of the nonzero bytes, the rest
 * of the row = -1, num[row] = n.  idx is rows x NK. */
int bsa_oracle_mask_to_lut(const int8_t* mask, int64_t rows, int32_t NK,
                           int32_t* idx, int32_t* num);

/* Number of OpenMP threads the oracle will use. */
int bsa_oracle_num_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_ORACLE_H */
