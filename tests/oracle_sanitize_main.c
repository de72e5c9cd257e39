/*
 * oracle_sanitize_main.c -- drives every entry point of the CPU oracle
 * (oracle/bsa_oracle.c) on small inputs, for a build with
 * -fsanitize=address,undefined (tests/test_oracle_sanitize.py compiles and
 * runs it; test infrastructure only).
 *
 * Every buffer is allocated at exactly the size the oracle's contract
 * states, so that a read or write past it is reported.  The metadata holds
 * the cases the oracle must survive: counts below 0 and above max_kv, LUT
 * entries outside [0, NK) (including INT32_MIN / INT32_MAX) and repeated
 * below the count, garbage past the count, variable block sizes below 0,
 * 0 and above the block, all-zero mask rows, shared metadata rows (strides
 * 0), grouped-query heads, rectangular shapes, zero and negative fp8 block
 * scales, codebook-coded K/V, a subset of units, and arguments the oracle
 * must reject (a non-finite softmax scale).  Exit status 0 = every call
 * returned what it should; the sanitizers abort on any finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsa_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* xorshift64* (Vigna), a seeded source of test inputs only */
static uint64_t rnd(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

/* bf16 bit patterns of values in about [-2, 2] */
static uint16_t* bf16_buf(size_t n) {
  uint16_t* p = (uint16_t*)xmalloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) {
    float f = (float)((double)(rnd() >> 11) / 9007199254740992.0 * 4.0 - 2.0);
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    p[i] = (uint16_t)(w >> 16);
  }
  return p;
}

/* fp8 e4m3fn bytes, NaN codes (S.1111.111) avoided */
static uint8_t* fp8_buf(size_t n) {
  uint8_t* p = (uint8_t*)xmalloc(n);
  for (size_t i = 0; i < n; ++i) {
    uint8_t b = (uint8_t)rnd();
    if ((b & 0x7F) == 0x7F) b &= 0xF7;
    p[i] = b;
  }
  return p;
}

static uint8_t* byte_buf(size_t n) {
  uint8_t* p = (uint8_t*)xmalloc(n);
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd();
  return p;
}

static float* f32_buf(size_t n, double lo, double hi) {
  float* p = (float*)xmalloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i)
    p[i] = (float)(lo + (hi - lo) * (double)(rnd() >> 11) / 9007199254740992.0);
  return p;
}

static int all_finite(const double* x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

/* Metadata of one LUT launch with every defensive case in it. */
typedef struct {
  int32_t* idx;
  int32_t* num;
  int32_t max_kv;
  int64_t rows;
} lut_meta;

static lut_meta make_lut(int64_t rows, int32_t NK, int32_t max_kv) {
  lut_meta m;
  m.rows = rows;
  m.max_kv = max_kv;
  m.idx = (int32_t*)xmalloc((size_t)(rows * max_kv) * sizeof(int32_t));
  m.num = (int32_t*)xmalloc((size_t)rows * sizeof(int32_t));
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t j = 0; j < max_kv; ++j) {
      int32_t v;
      switch (rnd() % 8) {
        case 0: v = -1; break;
        case 1: v = NK + (int32_t)(rnd() % 5); break;  /* past the last block */
        case 2: v = (rnd() & 1) ? INT32_MIN : INT32_MAX; break;
        default: v = (int32_t)(rnd() % (uint64_t)NK); break; /* repeats likely */
      }
      m.idx[r * max_kv + j] = v;
    }
    switch (r % 5) {
      case 0: m.num[r] = 0; break;
      case 1: m.num[r] = -3; break;
      case 2: m.num[r] = max_kv + 7; break;
      default: m.num[r] = (int32_t)(rnd() % (uint64_t)(max_kv + 1)); break;
    }
  }
  return m;
}

static int32_t* make_vbs(int32_t NK, int32_t block) {
  int32_t* v = (int32_t*)xmalloc((size_t)NK * sizeof(int32_t));
  for (int32_t i = 0; i < NK; ++i) {
    switch (i % 6) {
      case 0: v[i] = block; break;
      case 1: v[i] = 0; break;
      case 2: v[i] = -4; break;
      case 3: v[i] = block + 9; break;
      default: v[i] = 1 + (int32_t)(rnd() % (uint64_t)block); break;
    }
  }
  return v;
}

/* Forward over every kv encoding, both forms, all units and a subset. */
static void forward_cases(void) {
  const int32_t B = 2, H = 4, Hk = 2, D = 128, block = 64;
  const int32_t Sq = 3 * block, Sk = 5 * block;
  const int32_t NQ = Sq / block, NK = Sk / block;
  const size_t nq = (size_t)B * H * Sq * D, nkv = (size_t)B * Hk * Sk * D;
  const int64_t total = (int64_t)B * H * NQ;
  uint16_t* q = bf16_buf(nq);
  int32_t* vbs = make_vbs(NK, block);
  lut_meta lut = make_lut(total, NK, 6);
  int8_t* mask = (int8_t*)xmalloc((size_t)(total * NK));
  for (int64_t i = 0; i < total * NK; ++i) mask[i] = (int8_t)(rnd() % 3 == 0 ? rnd() : 0);
  for (int32_t kb = 0; kb < NK; ++kb) mask[kb] = 0; /* row 0 selects nothing */
  const size_t nscale = (size_t)B * Hk * NK;
  float* ks = f32_buf(nscale, -0.02, 0.02);
  float* vs = f32_buf(nscale, -0.02, 0.02);
  ks[0] = 0.f; /* an all-zero K block scale */
  vs[1] = 0.f;
  float* cb8 = f32_buf(256, -1.0, 1.0);
  float* cb4 = f32_buf(16, -1.0, 1.0);
  int64_t sub[3] = {total - 1, 0, 5};

  for (int kv = 0; kv <= 3; ++kv) {
    void* k;
    void* v;
    size_t kv_elems = kv == 3 ? nkv / 2 : nkv; /* packed i4: two codes a byte */
    if (kv == 0) {
      k = bf16_buf(kv_elems);
      v = bf16_buf(kv_elems);
    } else if (kv == 1) {
      k = fp8_buf(kv_elems);
      v = fp8_buf(kv_elems);
    } else {
      k = byte_buf(kv_elems);
      v = byte_buf(kv_elems);
    }
    const float* kcb = kv == 2 ? cb8 : kv == 3 ? cb4 : NULL;
    const float* vcb = kcb;
    for (int shared = 0; shared <= 1; ++shared) {
      const int64_t sb = shared ? 0 : (int64_t)H * NQ, sh = shared ? 0 : NQ;
      double* out = (double*)xmalloc(nq * sizeof(double));
      double* lse = (double*)xmalloc((size_t)B * H * Sq * sizeof(double));
      int rc = bsa_oracle_fwd_lut(q, k, v, kv, ks, vs, kcb, vcb, lut.idx, lut.num,
                                  lut.max_kv, sb, sh, vbs, 0.088, B, H, Hk, Sq,
                                  Sk, D, block, NULL, total, out, lse);
      expect(rc == 0, "fwd_lut all units");
      expect(all_finite(out, nq), "fwd_lut finite output");
      rc = bsa_oracle_fwd_bitmap(q, k, v, kv, ks, vs, kcb, vcb, mask, sb, sh, vbs,
                                 -0.5, B, H, Hk, Sq, Sk, D, block, NULL, total,
                                 out, lse);
      expect(rc == 0, "fwd_bitmap all units");
      expect(all_finite(out, nq), "fwd_bitmap finite output");
      free(out);
      free(lse);
      double* o3 = (double*)xmalloc((size_t)3 * block * D * sizeof(double));
      double* l3 = (double*)xmalloc((size_t)3 * block * sizeof(double));
      rc = bsa_oracle_fwd_lut(q, k, v, kv, ks, vs, kcb, vcb, lut.idx, lut.num,
                              lut.max_kv, sb, sh, NULL, 0.0, B, H, Hk, Sq, Sk, D,
                              block, sub, 3, o3, l3);
      expect(rc == 0, "fwd_lut unit subset, sm_scale 0");
      free(o3);
      free(l3);
    }
    free(k);
    free(v);
  }

  /* arguments the oracle rejects before writing anything */
  {
    double out1 = 7.0, lse1 = 7.0;
    uint16_t* k = bf16_buf(nkv);
    int64_t one = 0, bad = total;
    expect(bsa_oracle_fwd_lut(q, k, k, 0, NULL, NULL, NULL, NULL, lut.idx,
                              lut.num, lut.max_kv, (int64_t)H * NQ, NQ, vbs,
                              NAN, B, H, Hk, Sq, Sk, D, block, &one, 1, &out1,
                              &lse1) != 0,
           "NaN sm_scale rejected");
    expect(bsa_oracle_fwd_bitmap(q, k, k, 0, NULL, NULL, NULL, NULL, mask,
                                 (int64_t)H * NQ, NQ, vbs, INFINITY, B, H, Hk,
                                 Sq, Sk, D, block, &one, 1, &out1, &lse1) != 0,
           "infinite sm_scale rejected");
    expect(bsa_oracle_fwd_lut(q, k, k, 0, NULL, NULL, NULL, NULL, lut.idx,
                              lut.num, lut.max_kv, (int64_t)H * NQ, NQ, vbs,
                              0.1, B, H, Hk, Sq, Sk, D, block, &bad, 1, &out1,
                              &lse1) != 0,
           "unit past the end rejected");
    expect(bsa_oracle_fwd_lut(q, k, k, 0, NULL, NULL, NULL, NULL, lut.idx,
                              lut.num, lut.max_kv, (int64_t)H * NQ, NQ, vbs,
                              0.1, B, H, Hk, Sq, Sk, D, block, NULL, 1, &out1,
                              &lse1) != 0,
           "all units with a count other than B*H*NQ rejected");
    expect(out1 == 7.0 && lse1 == 7.0, "rejected calls write nothing");
    free(k);
  }

  /* integer decode */
  {
    int32_t* counts = (int32_t*)xmalloc((size_t)(total * NK) * sizeof(int32_t));
    expect(bsa_oracle_key_counts(0, lut.idx, lut.num, lut.max_kv, (int64_t)H * NQ,
                                 NQ, NULL, 0, 0, vbs, B, H, Sq, Sk, block, NULL,
                                 total, counts) == 0,
           "key_counts LUT");
    expect(bsa_oracle_key_counts(1, NULL, NULL, 0, 0, 0, mask, (int64_t)H * NQ, NQ,
                                 vbs, B, H, Sq, Sk, block, NULL, total, counts) == 0,
           "key_counts bitmap");
    for (int64_t i = 0; i < total * NK; ++i)
      expect(counts[i] >= 0 && counts[i] <= block, "count within [0, block]");
    free(counts);
  }

  free(q);
  free(vbs);
  free(lut.idx);
  free(lut.num);
  free(mask);
  free(ks);
  free(vs);
  free(cb8);
  free(cb4);
}

static void backward_cases(void) {
  const int32_t B = 1, H = 4, Hk = 2, D = 128, block = 64;
  const int32_t Sq = 2 * block, Sk = 4 * block;
  const int32_t NQ = Sq / block, NK = Sk / block;
  const size_t nq = (size_t)B * H * Sq * D, nkv = (size_t)B * Hk * Sk * D;
  const int64_t total = (int64_t)B * H * NQ;
  uint16_t* q = bf16_buf(nq);
  uint16_t* k = bf16_buf(nkv);
  uint16_t* v = bf16_buf(nkv);
  uint16_t* dout = bf16_buf(nq);
  int32_t* vbs = make_vbs(NK, block);
  lut_meta lut = make_lut(total, NK, 5);
  int8_t* mask = (int8_t*)xmalloc((size_t)(total * NK));
  for (int64_t i = 0; i < total * NK; ++i) mask[i] = (int8_t)(rnd() & 1);
  double* dq = (double*)xmalloc(nq * sizeof(double));
  double* dk = (double*)xmalloc(nkv * sizeof(double));
  double* dv = (double*)xmalloc(nkv * sizeof(double));
  expect(bsa_oracle_bwd(0, q, k, v, dout, lut.idx, lut.num, lut.max_kv, NULL,
                        (int64_t)H * NQ, NQ, vbs, 0.088, B, H, Hk, Sq, Sk, D,
                        block, dq, dk, dv) == 0,
         "bwd LUT");
  expect(all_finite(dq, nq) && all_finite(dk, nkv) && all_finite(dv, nkv),
         "bwd LUT finite");
  expect(bsa_oracle_bwd(1, q, k, v, dout, NULL, NULL, 0, mask, (int64_t)H * NQ, NQ,
                        NULL, -0.3, B, H, Hk, Sq, Sk, D, block, dq, dk, dv) == 0,
         "bwd bitmap");
  expect(bsa_oracle_bwd(0, q, k, v, dout, lut.idx, lut.num, lut.max_kv, NULL,
                        (int64_t)H * NQ, NQ, vbs, NAN, B, H, Hk, Sq, Sk, D,
                        block, dq, dk, dv) != 0,
         "bwd rejects NaN sm_scale");
  free(q);
  free(k);
  free(v);
  free(dout);
  free(vbs);
  free(lut.idx);
  free(lut.num);
  free(mask);
  free(dq);
  free(dk);
  free(dv);
}

static void decoder_and_compaction_cases(void) {
  for (uint32_t b = 0; b < 65536; ++b) {
    double x = bsa_oracle_bf16_value((uint16_t)b);
    (void)x;
  }
  int nan_codes = 0;
  for (uint32_t b = 0; b < 256; ++b) nan_codes += isnan(bsa_oracle_fp8e4m3_value((uint8_t)b));
  expect(nan_codes == 2, "two fp8 e4m3fn NaN codes");
  /* codebook indices of packed i4 (two per byte) and i8 codes */
  uint8_t packed[3] = {0x0F, 0x80, 0x7A};
  int8_t codes[2] = {-128, 127};
  expect(bsa_oracle_codebook_index(3, packed, 0) >= 0 &&
             bsa_oracle_codebook_index(3, packed, 5) < 16,
         "i4 index range");
  expect(bsa_oracle_codebook_index(2, codes, 0) == 0 &&
             bsa_oracle_codebook_index(2, codes, 1) == 255,
         "i8 index ends");
  const int64_t rows = 7;
  const int32_t NK = 70; /* not a multiple of any vector width */
  int8_t* mask = (int8_t*)xmalloc((size_t)(rows * NK));
  for (int64_t i = 0; i < rows * NK; ++i) mask[i] = (int8_t)(rnd() % 4 == 0 ? -1 : 0);
  memset(mask, 0, (size_t)NK);        /* an empty row */
  memset(mask + NK, 1, (size_t)NK);   /* a full row */
  int32_t* idx = (int32_t*)xmalloc((size_t)(rows * NK) * sizeof(int32_t));
  int32_t* num = (int32_t*)xmalloc((size_t)rows * sizeof(int32_t));
  expect(bsa_oracle_mask_to_lut(mask, rows, NK, idx, num) == 0, "mask_to_lut");
  expect(num[0] == 0 && num[1] == NK, "mask_to_lut counts");
  free(mask);
  free(idx);
  free(num);
}

int main(void) {
  decoder_and_compaction_cases();
  forward_cases();
  backward_cases();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: all calls checked\n");
  return 0;
}
