/*
 * bsa_oracle.c -- plain, slow CPU oracle for block-sparse attention forward.
 *
 * TEST INFRASTRUCTURE ONLY (see bsa_oracle.h): used by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark; never by the product path.
 *
 * Every step is the plain definition written out in double precision:
 * decode the selected key set of a work unit, list its attended keys in
 * ascending order, then for each query row take the dot products, the
 * base-2 softmax over the attended keys (two passes: max, then weights) and
 * the weighted sum of values.  No blocking, fusion or online rescaling.
 * OpenMP only spreads independent work units over cores.
 */
#include "bsa_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoders ----------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32: the value is exact. */
double bsa_oracle_bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 "fn" encoding: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 is subnormal
 * (2^-6 * m/8); no infinities; S.1111.111 is NaN; largest finite 448.
 * The K/V quantisation recipe (scale = amax/448) fixes this encoding. */
double bsa_oracle_fp8e4m3_value(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 0xF;
  int m = byte & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* ---- selected set of one work unit ----------------------------------- */

static int32_t clamp_i32(int32_t x, int32_t lo, int32_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

/* LUT form: sel[kb] = 1 for every idx[row, j], j < clamp(num,0,max_kv),
 * with 0 <= idx < NK.  Entries at j >= count are never read; order and
 * repetitions do not matter (a set). */
static void select_lut(const int32_t* q2k_idx, const int32_t* q2k_num,
                       int32_t max_kv, int64_t row, int32_t NK,
                       unsigned char* sel) {
  int32_t n = clamp_i32(q2k_num[row], 0, max_kv);
  memset(sel, 0, (size_t)NK);
  for (int32_t j = 0; j < n; ++j) {
    int32_t kb = q2k_idx[row * (int64_t)max_kv + j];
    if (kb >= 0 && kb < NK) sel[kb] = 1;
  }
}

/* Bitmap form: nonzero byte = attend. */
static void select_bitmap(const int8_t* mask, int64_t row, int32_t NK,
                          unsigned char* sel) {
  for (int32_t kb = 0; kb < NK; ++kb)
    sel[kb] = mask[row * (int64_t)NK + kb] != 0;
}

/* Number of valid keys of key block kb. */
static int32_t block_valid(const int32_t* vbs, int32_t kb, int32_t block) {
  return vbs ? clamp_i32(vbs[kb], 0, block) : block;
}

/* ---- attention over the attended set of one unit --------------------- */

typedef struct {
  const uint16_t* q;
  const void* k;
  const void* v;
  int kv_dtype;
  const float* k_scale;
  const float* v_scale;
  const float* k_codebook; /* codebook modes: 256 (i8) or 16 (i4) entries */
  const float* v_codebook;
  const int32_t* vbs;
  double sm_scale;
  int32_t H, Hk;  /* query heads, key/value heads (H a multiple of Hk) */
  int32_t Sq, Sk; /* query and key sequence lengths */
  int32_t D, block;
} attn_args;

/* Codebook index of element `elem` of a codebook-coded tensor (rocke
 * "sage_attention.py", codebook-dequant primitives): i8 codes index a
 * 256-entry table at code + 128; i4 codes are packed two per byte, element
 * 2i in the low nibble and 2i+1 in the high nibble (two's complement in
 * [-8, 7]), and index a 16-entry table at code + 8. */
int bsa_oracle_codebook_index(int kv_dtype, const void* base, int64_t elem) {
  if (kv_dtype == ORACLE_KV_I8_CODEBOOK)
    return (int)((const int8_t*)base)[elem] + 128;
  const uint8_t byte = ((const uint8_t*)base)[elem >> 1];
  const int nib = (elem & 1) ? (byte >> 4) : (byte & 15);
  return (nib >= 8 ? nib - 16 : nib) + 8;
}

static double kv_value(const attn_args* a, const void* base, const float* scale,
                       const float* codebook, int64_t elem, int64_t scale_idx) {
  switch (a->kv_dtype) {
    case ORACLE_KV_BF16:
      return bsa_oracle_bf16_value(((const uint16_t*)base)[elem]);
    case ORACLE_KV_FP8E4M3:
      return bsa_oracle_fp8e4m3_value(((const uint8_t*)base)[elem]) *
             (double)scale[scale_idx];
    default: /* codebook value times the block scale */
      return (double)codebook[bsa_oracle_codebook_index(a->kv_dtype, base, elem)] *
             (double)scale[scale_idx];
  }
}

/* Computes the `block` output rows of unit (b, h, qb) given its selected set.
 * Query head h reads key/value head h / (H/Hk): consecutive query heads
 * share one K/V head (rocke "sparse_attention.py": separate query and KV
 * head counts, a KV head index per head).  The steps follow the definition
 * in order: list the attended keys ascending; decode each attended key and
 * value once into real numbers (rocke "sage_attention.py", module docstring:
 * K/V are dequantised per block before the score and the PV product); then,
 * per query row, the scores, their maximum, the weights, their sum, the
 * weighted sum of values and the LSE.  keys and t are scratch arrays of
 * length Sk, qd of length D.  Returns nonzero if the decoded-key buffers
 * cannot be allocated. */
static int attend_unit(const attn_args* a, int32_t b, int32_t h, int32_t qb,
                       const unsigned char* sel, int64_t* keys, double* t,
                       double* qd, double* out, double* lse) {
  const int32_t D = a->D, block = a->block, NK = a->Sk / block;
  const int64_t qplane = ((int64_t)b * a->H + h) * (int64_t)a->Sq * D;
  const int64_t kvhead = (int64_t)b * a->Hk + h / (a->H / a->Hk);
  const int64_t plane = kvhead * (int64_t)a->Sk * D;
  const double c = a->sm_scale / log(2.0); /* sm_scale * log2(e) */

  /* attended keys, ascending */
  int64_t n_att = 0;
  for (int32_t kb = 0; kb < NK; ++kb) {
    if (!sel[kb]) continue;
    int32_t nv = block_valid(a->vbs, kb, block);
    for (int32_t tt = 0; tt < nv; ++tt) keys[n_att++] = (int64_t)kb * block + tt;
  }

  /* decoded keys kd[j][d] and values vd[j][d] of the attended keys */
  double* kd = NULL;
  double* vd = NULL;
  if (n_att > 0) {
    kd = (double*)malloc(sizeof(double) * (size_t)n_att * (size_t)D);
    vd = (double*)malloc(sizeof(double) * (size_t)n_att * (size_t)D);
    if (!kd || !vd) {
      free(kd);
      free(vd);
      return 1;
    }
    for (int64_t j = 0; j < n_att; ++j) {
      const int64_t key = keys[j];
      const int64_t srow = kvhead * NK + key / block;
      for (int32_t d = 0; d < D; ++d) {
        kd[j * D + d] = kv_value(a, a->k, a->k_scale, a->k_codebook,
                                 plane + key * D + d, srow);
        vd[j * D + d] = kv_value(a, a->v, a->v_scale, a->v_codebook,
                                 plane + key * D + d, srow);
      }
    }
  }

  for (int32_t r = 0; r < block; ++r) {
    double* o = out + (int64_t)r * D;
    const int64_t qrow = qplane + ((int64_t)qb * block + r) * D;
    if (n_att == 0) {
      for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
      lse[r] = -(double)FLT_MAX;
      continue;
    }
    for (int32_t d = 0; d < D; ++d) qd[d] = bsa_oracle_bf16_value(a->q[qrow + d]);
    /* pass 1: scaled scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_att; ++j) {
      double s = 0.0;
      for (int32_t d = 0; d < D; ++d) s += qd[d] * kd[j * D + d];
      t[j] = s * c;
      if (t[j] > m) m = t[j];
    }
    /* pass 2: weights, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < n_att; ++j) {
      const double w = exp2(t[j] - m);
      l += w;
      for (int32_t d = 0; d < D; ++d) o[d] += w * vd[j * D + d];
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= l;
    lse[r] = m + log2(l);
  }
  free(kd);
  free(vd);
  return 0;
}

/* ---- argument checks shared by the entry points ---------------------- */

/* The softmax scale may be any finite value (zero: equal weights;
 * negative: reversed ranking); NaN and infinities are rejected, as by the
 * GPU entry points. */
static int check_scale(double sm_scale) { return isfinite(sm_scale) ? 0 : 1; }

static int check_dims(int32_t B, int32_t H, int32_t Hk, int32_t Sq,
                      int32_t Sk, int32_t D, int32_t block) {
  if (B <= 0 || H <= 0 || Hk <= 0 || Sq <= 0 || Sk <= 0 || D <= 0 || block <= 0)
    return 1;
  if (H % Hk != 0 || Sq % block != 0 || Sk % block != 0) return 1;
  return 0;
}

static int check_kv(int kv_dtype, const float* k_scale, const float* v_scale,
                    const float* k_codebook, const float* v_codebook,
                    int32_t D) {
  if (kv_dtype < ORACLE_KV_BF16 || kv_dtype > ORACLE_KV_I4_CODEBOOK) return 1;
  if (kv_dtype != ORACLE_KV_BF16 && (!k_scale || !v_scale)) return 1;
  if (kv_dtype >= ORACLE_KV_I8_CODEBOOK && (!k_codebook || !v_codebook)) return 1;
  if (kv_dtype == ORACLE_KV_I4_CODEBOOK && D % 2 != 0) return 1;
  return 0;
}

static int check_units(const int64_t* units, int64_t n_units, int64_t total) {
  if (!units) return n_units == total ? 0 : 1;
  for (int64_t i = 0; i < n_units; ++i)
    if (units[i] < 0 || units[i] >= total) return 1;
  return 0;
}

enum { FORM_LUT = 0, FORM_BITMAP = 1 };

typedef struct {
  int form;
  const int32_t* q2k_idx;
  const int32_t* q2k_num;
  int32_t max_kv;
  int64_t sb, sh; /* metadata row strides (in rows) */
  const int8_t* mask;
} sel_args;

static void unit_select(const sel_args* s, int32_t b, int32_t h, int32_t qb,
                        int32_t NK, unsigned char* sel) {
  const int64_t row = (int64_t)b * s->sb + (int64_t)h * s->sh + qb;
  if (s->form == FORM_LUT)
    select_lut(s->q2k_idx, s->q2k_num, s->max_kv, row, NK, sel);
  else
    select_bitmap(s->mask, row, NK, sel);
}

static int run_fwd(const attn_args* a, const sel_args* s, int32_t B,
                   const int64_t* units, int64_t n_units, double* out,
                   double* lse) {
  const int32_t NQ = a->Sq / a->block, NK = a->Sk / a->block;
  int failed = 0;
#pragma omp parallel
  {
    unsigned char* sel = (unsigned char*)malloc((size_t)NK);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)a->Sk);
    double* t = (double*)malloc(sizeof(double) * (size_t)a->Sk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)a->D);
    const int ok = sel && keys && t && qd;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_units; ++i) {
      if (!ok) continue;
      const int64_t u = units ? units[i] : i;
      const int32_t qb = (int32_t)(u % NQ);
      const int32_t h = (int32_t)((u / NQ) % a->H);
      const int32_t b = (int32_t)(u / ((int64_t)NQ * a->H));
      unit_select(s, b, h, qb, NK, sel);
      if (attend_unit(a, b, h, qb, sel, keys, t, qd,
                      out + i * (int64_t)a->block * a->D,
                      lse + i * (int64_t)a->block)) {
#pragma omp atomic write
        failed = 1;
      }
    }
    free(sel);
    free(keys);
    free(t);
    free(qd);
  }
  (void)B;
  return failed ? 3 : 0;
}

/* ---- entry points ---------------------------------------------------- */

int bsa_oracle_fwd_lut(const uint16_t* q, const void* k, const void* v,
                       int kv_dtype, const float* k_scale, const float* v_scale,
                       const float* k_codebook, const float* v_codebook,
                       const int32_t* q2k_idx, const int32_t* q2k_num,
                       int32_t max_kv, int64_t meta_stride_b,
                       int64_t meta_stride_h, const int32_t* vbs,
                       double sm_scale, int32_t B, int32_t H, int32_t Hk,
                       int32_t Sq, int32_t Sk, int32_t D, int32_t block,
                       const int64_t* units, int64_t n_units, double* out,
                       double* lse) {
  if (!q || !k || !v || !q2k_idx || !q2k_num || !out || !lse) return 1;
  if (check_dims(B, H, Hk, Sq, Sk, D, block) || max_kv < 1) return 1;
  if (check_scale(sm_scale)) return 1;
  if (check_kv(kv_dtype, k_scale, v_scale, k_codebook, v_codebook, D)) return 1;
  if (check_units(units, n_units, (int64_t)B * H * (Sq / block))) return 1;
  attn_args a = {q, k, v, kv_dtype, k_scale, v_scale, k_codebook, v_codebook,
                 vbs, sm_scale, H, Hk, Sq, Sk, D, block};
  sel_args s = {FORM_LUT, q2k_idx, q2k_num, max_kv, meta_stride_b,
                meta_stride_h, NULL};
  return run_fwd(&a, &s, B, units, n_units, out, lse);
}

int bsa_oracle_fwd_bitmap(const uint16_t* q, const void* k, const void* v,
                          int kv_dtype, const float* k_scale,
                          const float* v_scale, const float* k_codebook,
                          const float* v_codebook, const int8_t* mask,
                          int64_t mask_stride_b, int64_t mask_stride_h,
                          const int32_t* vbs, double sm_scale, int32_t B,
                          int32_t H, int32_t Hk, int32_t Sq, int32_t Sk,
                          int32_t D, int32_t block, const int64_t* units,
                          int64_t n_units, double* out, double* lse) {
  if (!q || !k || !v || !mask || !out || !lse) return 1;
  if (check_dims(B, H, Hk, Sq, Sk, D, block)) return 1;
  if (check_scale(sm_scale)) return 1;
  if (check_kv(kv_dtype, k_scale, v_scale, k_codebook, v_codebook, D)) return 1;
  if (check_units(units, n_units, (int64_t)B * H * (Sq / block))) return 1;
  attn_args a = {q, k, v, kv_dtype, k_scale, v_scale, k_codebook, v_codebook,
                 vbs, sm_scale, H, Hk, Sq, Sk, D, block};
  sel_args s = {FORM_BITMAP, NULL, NULL, 0, mask_stride_b, mask_stride_h,
                mask};
  return run_fwd(&a, &s, B, units, n_units, out, lse);
}

int bsa_oracle_key_counts(int form, const int32_t* q2k_idx,
                          const int32_t* q2k_num, int32_t max_kv,
                          int64_t meta_stride_b, int64_t meta_stride_h,
                          const int8_t* mask, int64_t mask_stride_b,
                          int64_t mask_stride_h, const int32_t* vbs, int32_t B,
                          int32_t H, int32_t Sq, int32_t Sk, int32_t block,
                          const int64_t* units, int64_t n_units,
                          int32_t* counts) {
  if (!counts || check_dims(B, H, H, Sq, Sk, 1, block)) return 1;
  if (form == FORM_LUT && (!q2k_idx || !q2k_num || max_kv < 1)) return 1;
  if (form == FORM_BITMAP && !mask) return 1;
  if (form != FORM_LUT && form != FORM_BITMAP) return 1;
  const int32_t NQ = Sq / block, NK = Sk / block;
  if (check_units(units, n_units, (int64_t)B * H * NQ)) return 1;
  sel_args s;
  if (form == FORM_LUT) {
    sel_args t = {FORM_LUT, q2k_idx, q2k_num, max_kv, meta_stride_b,
                  meta_stride_h, NULL};
    s = t;
  } else {
    sel_args t = {FORM_BITMAP, NULL, NULL, 0, mask_stride_b, mask_stride_h,
                  mask};
    s = t;
  }
  unsigned char* sel = (unsigned char*)malloc((size_t)NK);
  if (!sel) return 3;
  for (int64_t i = 0; i < n_units; ++i) {
    const int64_t u = units ? units[i] : i;
    const int32_t qb = (int32_t)(u % NQ);
    const int32_t h = (int32_t)((u / NQ) % H);
    const int32_t b = (int32_t)(u / ((int64_t)NQ * H));
    unit_select(&s, b, h, qb, NK, sel);
    for (int32_t kb = 0; kb < NK; ++kb)
      counts[i * (int64_t)NK + kb] = sel[kb] ? block_valid(vbs, kb, block) : 0;
  }
  free(sel);
  return 0;
}

/* ---- backward pass (gradients of the forward definition) ------------- */

/* For one work unit, the plain chain rule of softmax attention over the
 * unit's attended keys, in natural-log units (the base-2 form of the forward
 * pass is the same function):
 *   s_j  = sm_scale * (q_r . k_j),  p_j = e^(s_j - m) / sum_i e^(s_i - m)
 *   O_r  = sum_j p_j v_j
 *   dv_j += p_j dO_r
 *   dp_j  = dO_r . v_j,   delta = sum_j p_j dp_j  (= dO_r . O_r)
 *   ds_j  = p_j (dp_j - delta)
 *   dq_r  = sm_scale * sum_j ds_j k_j,   dk_j += sm_scale * ds_j q_r
 * A row with no attended key has no dependence on K or V and dq_r = 0.
 * K/V head kvh = h / (H/Hk) receives the gradients of all its query heads. */
static void backward_unit(const attn_args* a, const uint16_t* dout, int32_t b,
                          int32_t h, int32_t qb, const unsigned char* sel,
                          int64_t* keys, double* s, double* dp, double* qd,
                          double* dod, double* dq, double* dk, double* dv) {
  const int32_t D = a->D, block = a->block, NK = a->Sk / block;
  const int64_t qplane = ((int64_t)b * a->H + h) * (int64_t)a->Sq * D;
  const int64_t kvhead = (int64_t)b * a->Hk + h / (a->H / a->Hk);
  const int64_t plane = kvhead * (int64_t)a->Sk * D;

  int64_t n_att = 0;
  for (int32_t kb = 0; kb < NK; ++kb) {
    if (!sel[kb]) continue;
    int32_t nv = block_valid(a->vbs, kb, block);
    for (int32_t tt = 0; tt < nv; ++tt) keys[n_att++] = (int64_t)kb * block + tt;
  }
  if (n_att == 0) return; /* dq rows stay 0 */

  for (int32_t r = 0; r < block; ++r) {
    const int64_t qrow = qplane + ((int64_t)qb * block + r) * D;
    for (int32_t d = 0; d < D; ++d) {
      qd[d] = bsa_oracle_bf16_value(a->q[qrow + d]);
      dod[d] = bsa_oracle_bf16_value(dout[qrow + d]);
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n_att; ++j) {
      const int64_t krow = plane + keys[j] * D;
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d)
        acc += qd[d] * bsa_oracle_bf16_value(((const uint16_t*)a->k)[krow + d]);
      s[j] = acc * a->sm_scale;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_att; ++j) {
      s[j] = exp(s[j] - m); /* unnormalised weight */
      l += s[j];
    }
    double delta = 0.0;
    for (int64_t j = 0; j < n_att; ++j) {
      const int64_t vrow = plane + keys[j] * D;
      s[j] /= l; /* p_j */
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d)
        acc += dod[d] * bsa_oracle_bf16_value(((const uint16_t*)a->v)[vrow + d]);
      dp[j] = acc;
      delta += s[j] * acc;
    }
    double* dqr = dq + qrow;
    for (int64_t j = 0; j < n_att; ++j) {
      const int64_t row = plane + keys[j] * D;
      const double ds = s[j] * (dp[j] - delta);
      for (int32_t d = 0; d < D; ++d) {
        dqr[d] += a->sm_scale * ds *
                  bsa_oracle_bf16_value(((const uint16_t*)a->k)[row + d]);
        dk[row + d] += a->sm_scale * ds * qd[d];
        dv[row + d] += s[j] * dod[d];
      }
    }
  }
}

int bsa_oracle_bwd(int form, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, const uint16_t* dout,
                   const int32_t* q2k_idx, const int32_t* q2k_num,
                   int32_t max_kv, const int8_t* mask, int64_t meta_stride_b,
                   int64_t meta_stride_h, const int32_t* vbs, double sm_scale,
                   int32_t B, int32_t H, int32_t Hk, int32_t Sq, int32_t Sk,
                   int32_t D, int32_t block, double* dq, double* dk,
                   double* dv) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
  if (check_dims(B, H, Hk, Sq, Sk, D, block)) return 1;
  if (check_scale(sm_scale)) return 1;
  if (form == FORM_LUT && (!q2k_idx || !q2k_num || max_kv < 1)) return 1;
  if (form == FORM_BITMAP && !mask) return 1;
  if (form != FORM_LUT && form != FORM_BITMAP) return 1;
  attn_args a = {q, k, v, ORACLE_KV_BF16, NULL, NULL, NULL, NULL, vbs,
                 sm_scale, H, Hk, Sq, Sk, D, block};
  sel_args s;
  if (form == FORM_LUT) {
    sel_args t = {FORM_LUT, q2k_idx, q2k_num, max_kv, meta_stride_b,
                  meta_stride_h, NULL};
    s = t;
  } else {
    sel_args t = {FORM_BITMAP, NULL, NULL, 0, meta_stride_b, meta_stride_h,
                  mask};
    s = t;
  }
  const int32_t NQ = Sq / block, NK = Sk / block, G = H / Hk;
  memset(dq, 0, sizeof(double) * (size_t)B * H * Sq * D);
  memset(dk, 0, sizeof(double) * (size_t)B * Hk * Sk * D);
  memset(dv, 0, sizeof(double) * (size_t)B * Hk * Sk * D);
  int failed = 0;
  /* one (batch, K/V head) group per iteration: it owns its dk/dv rows and
   * the dq rows of its query heads */
#pragma omp parallel
  {
    unsigned char* sel = (unsigned char*)malloc((size_t)NK);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)Sk);
    double* sv = (double*)malloc(sizeof(double) * (size_t)Sk);
    double* dpv = (double*)malloc(sizeof(double) * (size_t)Sk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* dod = (double*)malloc(sizeof(double) * (size_t)D);
    const int ok = sel && keys && sv && dpv && qd && dod;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t grp = 0; grp < (int64_t)B * Hk; ++grp) {
      if (!ok) continue;
      const int32_t b = (int32_t)(grp / Hk), kvh = (int32_t)(grp % Hk);
      for (int32_t h = kvh * G; h < (kvh + 1) * G; ++h)
        for (int32_t qb = 0; qb < NQ; ++qb) {
          unit_select(&s, b, h, qb, NK, sel);
          backward_unit(&a, dout, b, h, qb, sel, keys, sv, dpv, qd, dod, dq,
                        dk, dv);
        }
    }
    free(sel);
    free(keys);
    free(sv);
    free(dpv);
    free(qd);
    free(dod);
  }
  return failed ? 3 : 0;
}

int bsa_oracle_mask_to_lut(const int8_t* mask, int64_t rows, int32_t NK,
                           int32_t* idx, int32_t* num) {
  if (!mask || !idx || !num || rows < 0 || NK <= 0) return 1;
  for (int64_t r = 0; r < rows; ++r) {
    int32_t n = 0;
    for (int32_t kb = 0; kb < NK; ++kb)
      if (mask[r * (int64_t)NK + kb] != 0) idx[r * (int64_t)NK + n++] = kb;
    for (int32_t j = n; j < NK; ++j) idx[r * (int64_t)NK + j] = -1;
    num[r] = n;
  }
  return 0;
}

int bsa_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
