// bsa_fwd.hip -- block-sparse attention forward for MI355X (gfx950 / CDNA4).
//
// One workgroup computes one work unit: the `BLK` query rows of query block
// qb of head h of batch b.  In a short launch (block 64, bf16 K/V, at most
// BSA_FWD_KEY_SPLIT_MAX_UNITS units) the workgroup holds two groups of waves
// that each sweep part of the unit's selected blocks for the same query
// rows; their partial results are merged before A8.  The steps, in order:
//
//  A1  unit id -> (b, h, qb), with workgroups of consecutive ids spread so
//      that each XCD (and its L2) serves a contiguous range of heads.  The
//      unit may take qb from a launch order (bsa_fwd_lut_ordered,
//      bsa_fwd_bitmap_ordered; the order pass in bsa_order.hip ranks each
//      head's units heaviest first,
//      so units of similar length run side by side and stay at the same
//      point of their key sweeps, sharing K/V in L2).  Query head h reads
//      K/V head h / (H/Hk) (grouped-query attention; rocke
//      "sparse_attention.py" keeps separate query and KV head counts and
//      query and key lengths, both supported here).
//  A2  selected-set decode into LDS.  LUT form: the row's first
//      clamp(num, 0, max_kv) entries are scattered into a byte map
//      (duplicate stores write the same value, out-of-range entries are
//      dropped), as in rocke "sparse_attention.py" `_stage_vsa_bitmap_to_lds`;
//      a selected block's byte holds its valid key count.  Bitmap form: the
//      mask row is copied into the same LDS map (`_stage_jenga_mask_to_lds`
//      on the same page).  One wave then
//      compacts the bitmap into an ascending list of selected key blocks that
//      have at least one valid key (ballot + popcount), so the K loop runs
//      over selected tiles only and never touches an unselected one (the
//      tile-skipping form the page calls strictly stronger than forcing
//      -inf).  Ascending order makes the result independent of LUT order,
//      padding and repetitions.
//  A3  Q: each wave keeps its 32 query rows in VGPRs as MFMA operands for
//      the whole K loop (loaded once with 128-bit loads, issued before the
//      decode so that they arrive during it).
//  A4  K/V gather in 32-key tiles, only rows below a block's valid count
//      are read (direct global->LDS 128-bit loads).  bf16 K/V: the valid
//      keys of the selected blocks, in list order, are cut into tiles as
//      one stream, so a tile may draw rows from several blocks and only the
//      unit's last tile is partial (with valid counts below the block size
//      this removes the padded tail of every block).  With per-block scales
//      (fp8, scaled bf16) each tile stays inside one block.  Lanes of rows
//      past a tile's count re-read row 0 (fp8 writes zeros there), so every
//      row of every staged tile is written before it is read.  Tiles
//      are double-buffered in LDS: the loads of tile i+1 are in flight
//      while tile i is computed.  fp8 e4m3 K/V are widened to bf16 exactly
//      on the way into LDS.
//  A5  S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (fp32 accumulate), scaled by
//      c = sm_scale*log2(e) (times the block's K scale for fp8): t = s*c.
//  A6  softmax in exp2 form.  The reference m of each row is the maximum of
//      t over the valid keys of the unit's first tile and stays fixed (no
//      per-tile max or rescale); exponents are t - m, set to -inf for keys
//      at or past the block's valid count, so a masked key weighs exactly 0
//      for any sign of c.  If a weight or sum overflowed, the unit is
//      recomputed with the running-max / rescale scheme (vLLM "tq_decode"
//      step F shows it).
//      Partial sums l are kept per lane and reduced across the four lane
//      groups that share a query once, at the end.
//  A7  O^T += V^T P^T on the same MFMA; P is the softmax tile rounded to
//      bf16 (times the block's V scale for fp8), already in the operand
//      layout; V^T comes from the hardware transposing LDS read
//      ds_read_b64_tr_b16 (the gfx950 idiom of the "tq_decode" page).
//  A8  epilogue: O = acc / l rounded to bf16 (RNE), LSE = m + log2(l); a
//      unit with no attended key writes +0 and BSA_LSE_EMPTY (FastVideo
//      "block_sparse_attn_sm100a.py", `is_supported` docstring).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"
#include "bsa_device.h"

namespace {

constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // one K tile + one V tile
constexpr int NSTAGE = 2;

struct FwdParams {
  const uint16_t* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* idx;   // LUT form
  const int32_t* num;   // LUT form
  const int32_t* order; // LUT form: q-block launch order per (b, h), or null
  const int8_t* mask;   // bitmap form
  int64_t meta_sb;      // metadata row stride per batch (rows)
  int64_t meta_sh;      // metadata row stride per head (rows)
  const int32_t* vbs;   // [NK] or null
  uint16_t* out;
  float* lse;           // or null
  float c;              // sm_scale * log2(e)
  int32_t max_kv;
  int32_t H;            // query heads
  int32_t group;        // query heads per K/V head (H / Hk)
  int32_t Hk;           // key/value heads
  int32_t S, Sk;        // query and key sequence lengths
  int32_t NQ, NK;       // query blocks, key blocks
  int32_t n_units;
};

// LDS tile layout: 32 rows of 256 B, 16-byte chunks XOR-swizzled per row so
// that the MFMA operand reads are free of bank conflicts without padding.
// K tiles are read row-wise (16 rows x one chunk per 16 lanes): chunk c of
// row r sits at position c ^ (r & 15).  V tiles are read through the
// transposing LDS read (8 rows x 4 half-chunks per 32 lanes): position
// c ^ ((r & 7) << 1).
__device__ __forceinline__ int k_off(int r, int c) {
  return r * ROWB + ((c ^ (r & 15)) << 4);
}
__device__ __forceinline__ int v_off(int r, int c) {
  return r * ROWB + ((c ^ ((r & 7) << 1)) << 4);
}

// 4 fp8 e4m3 codes -> 4 bf16 (exact widening; scale 1).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t,
                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t,
                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

// fp8 K/V: 16 codes per 16-byte load, widened to bf16 in registers and
// stored into the same swizzled bf16 layout.
template <int NT>
struct Fp8Staging {
  static constexpr int CHUNKS = KT * 8;  // 32 rows x 8 chunks of 16 codes
  static constexpr int PER_THREAD = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly");
  u32x4 kr[PER_THREAD];
  u32x4 vr[PER_THREAD];
};

template <int NT>
__device__ __forceinline__ void load_tile_fp8(Fp8Staging<NT>& st, const char* kg,
                                              const char* vg, int nvt, int tid) {
#pragma unroll
  for (int i = 0; i < Fp8Staging<NT>::PER_THREAD; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3;
    const int col = c & 7;
    if (r < nvt) {
      st.kr[i] = *(const u32x4*)(kg + r * HD + col * 16);
      st.vr[i] = *(const u32x4*)(vg + r * HD + col * 16);
    } else {
      st.kr[i] = u32x4{0, 0, 0, 0};
      st.vr[i] = u32x4{0, 0, 0, 0};
    }
  }
}

template <int NT>
__device__ __forceinline__ void store_tile_fp8(const Fp8Staging<NT>& st,
                                               char* stage, int tid) {
  char* ks = stage;
  char* vs = stage + TILE_BYTES;
#pragma unroll
  for (int i = 0; i < Fp8Staging<NT>::PER_THREAD; ++i) {
    const int c = tid + i * NT;
    const int r = c >> 3;
    const int col = c & 7;  // bf16 chunks 2*col and 2*col+1
    const u32x2 k0 = fp8x4_to_bf16x4(st.kr[i].x), k1 = fp8x4_to_bf16x4(st.kr[i].y);
    const u32x2 k2 = fp8x4_to_bf16x4(st.kr[i].z), k3 = fp8x4_to_bf16x4(st.kr[i].w);
    const u32x2 v0 = fp8x4_to_bf16x4(st.vr[i].x), v1 = fp8x4_to_bf16x4(st.vr[i].y);
    const u32x2 v2 = fp8x4_to_bf16x4(st.vr[i].z), v3 = fp8x4_to_bf16x4(st.vr[i].w);
    *(u32x4*)(ks + k_off(r, 2 * col)) = u32x4{k0.x, k0.y, k1.x, k1.y};
    *(u32x4*)(ks + k_off(r, 2 * col + 1)) = u32x4{k2.x, k2.y, k3.x, k3.y};
    *(u32x4*)(vs + v_off(r, 2 * col)) = u32x4{v0.x, v0.y, v1.x, v1.y};
    *(u32x4*)(vs + v_off(r, 2 * col + 1)) = u32x4{v2.x, v2.y, v3.x, v3.y};
  }
}

// Tile shapes of the K loop: FULL = 32 valid keys; PART = 1..31 valid keys
// (keys past the count masked; the second 16-key half's QK^T is skipped
// when it holds no valid key).
enum TileKind { FULL = 0, PART = 1 };

// Accumulator state of one wave: O^T tiles, per-row reference m (log2
// units, identical in the four lanes of a row) and per-lane partial sums l.
struct Acc {
  f32x4 o[8][2];
  float m[2];
  float l[2];
};

// K operands of one tile for this wave (A operand of S^T = K Q^T):
// k[h][kk] holds dims kk*32 + 8g .. +7 of tile key h*16 + r16.  All eight
// reads are issued together right after the tile is published, so their
// latency is paid once per tile.
struct KOps {
  bf16x8 k[2][4];
};

__device__ __forceinline__ void load_k(const char* sb, uint32_t kbase, KOps& ko) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      ko.k[h][kk] = *(const bf16x8*)(sb + (kbase ^ (kk << 6)) + h * 16 * ROWB);
}

// Raw scores of one tile for this wave: s[qt][e], e = 4*s2 + j is key
// s2*16 + 4g + j of the tile and query qt*16 + r16 (no masking here: the
// mask is applied in t-space, see tile_exponents).
template <int KIND>
__device__ __forceinline__ void tile_scores(const KOps& ko, const bf16x8 (&qreg)[2][4],
                                            int nvt, float (&s)[2][8]) {
  f32x4 sacc[2][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
      sacc[0][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          ko.k[0][kk], qreg[qt][kk], kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[0][qt],
          0, 0, 0);
  sacc[1][0] = sacc[1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (KIND == FULL || nvt > 16) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        sacc[1][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            ko.k[1][kk], qreg[qt][kk], sacc[1][qt], 0, 0, 0);
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[qt][e] = sacc[e >> 2][qt][e & 3];
}

// Is entry e of this lane a valid key of the tile?  (Lane limit
// lim = nvt - 4g; a FULL tile has every key valid.)
template <int KIND>
__device__ __forceinline__ bool key_valid(int e, int lim) {
  return KIND == FULL || (e >> 2) * 16 + (e & 3) < lim;
}

// Row maximum of the tile in t-space: max over the valid keys of t = s*cs
// (any sign of cs), reduced over the four lanes of each row.
template <int KIND>
__device__ __forceinline__ void tile_max(const float (&s)[2][8], float cs, int lim,
                                         float (&tm)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      t[e] = key_valid<KIND>(e, lim) ? s[qt][e] * cs : -INFINITY;
    const float m0 = max3f(t[0], t[1], t[2]);
    const float m1 = max3f(t[3], t[4], t[5]);
    const float m2 = max3f(t[6], t[7], m0);
    tm[qt] = group_max(fmaxf(m1, m2));
  }
}

// Exponents of the tile's weights in place: s <- s*cs - m, and -inf for keys
// at or past the valid count, so that a masked key's weight is exactly 0
// whatever the sign of cs (cs = 0 included).
template <int KIND>
__device__ __forceinline__ void tile_exponents(float (&s)[2][8], float cs, int lim,
                                               const Acc& acc) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float nm = -acc.m[qt];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = __builtin_fmaf(s[qt][e], cs, nm);
      s[qt][e] = key_valid<KIND>(e, lim) ? x : -INFINITY;
    }
  }
}

// P = 2^x from the exponents of tile_exponents (zero for masked keys),
// added to the partial row sums, scaled by vsc (fp8 V scale) and packed to
// bf16 in the PV operand layout.
template <bool SCALE_P>
__device__ __forceinline__ void tile_probs(const float (&x)[2][8], float vsc, Acc& acc,
                                           bf16x8 (&pop)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(x[qt][e]);
    acc.l[qt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) +
                 ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    if constexpr (SCALE_P) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] *= vsc;
    }
    const u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                      pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    pop[qt] = __builtin_bit_cast(bf16x8, pk);
  }
}

// V^T operands of one tile: v[dt] holds, for d-row dt*16 + r16 of V^T, the
// tile keys of MFMA K index 8g+i: key 4g+i (i<4) and 16+4g+(i-4) (i>=4),
// matching P's accumulator layout.  Read with the transposing LDS read at
// vbase ^ (dt << 5) (+16 rows); issued before the softmax so that their
// latency hides under it.
struct VOps {
  bf16x8 v[8];
};

__device__ __forceinline__ void load_v(const char* sb, uint32_t vbase, VOps& vo) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint32_t va = vbase ^ (uint32_t)(dt << 5);
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sb + va));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(sb + va + 16 * ROWB));
    const i16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    vo.v[dt] = __builtin_bit_cast(bf16x8, vv);
  }
}

// O^T[d][query] += V^T P^T.
__device__ __forceinline__ void tile_pv(const VOps& vo, const bf16x8 (&pop)[2], Acc& acc) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
      acc.o[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo.v[dt], pop[qt],
                                                               acc.o[dt][qt], 0, 0, 0);
}

// Direct loads of this wave's share of a bf16 tile.  The tile's 8 slices
// of 4 rows (1 KB) are dealt round-robin to the NW waves: slice
// j = wave + i*NW lands at LDS stage + j*1024 (K) and stage + TILE_BYTES +
// j*1024 (V); lane l fills LDS position l & 15 of row 4j + l/16 with the
// chunk the swizzle places there, read from global offset ko[i] / vo[i]
// (row offset and swizzle folded in, fixed per lane).  In a tile with
// nvt < 32 valid rows, lanes of rows at or past nvt re-read the chunk at the
// same position of the tile's row 0 instead (always a valid key; the row is
// masked to -inf in the scores and meets a zero weight in PV), so the load
// count never depends on nvt and no row past the block's valid count is read.
template <int NW>
__device__ __forceinline__ void issue_bf16(const char* kg, const char* vg,
                                           uint32_t kdst, uint32_t vdst,
                                           const uint32_t (&ko)[8 / NW],
                                           const uint32_t (&vo)[8 / NW], int wave,
                                           int l4, int nvt) {
  if (nvt >= KT) {
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const uint32_t j = (uint32_t)(wave + i * NW);
      dma16(kg, ko[i], kdst + j * 1024u);
      dma16(vg, vo[i], vdst + j * 1024u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const int j = wave + i * NW;
      const bool ok = 4 * j + l4 < nvt;
      dma16(kg, ok ? ko[i] : (ko[i] & 0xFFu), kdst + (uint32_t)j * 1024u);
      dma16(vg, ok ? vo[i] : (vo[i] & 0xFFu), vdst + (uint32_t)j * 1024u);
    }
  }
}

// Waves per SIMD the register budget is sized for.  A 128-row unit runs 4
// waves in 32 KB of LDS, so LDS would allow 4 per SIMD; capping registers
// at 168 gives 3 (bf16 only: the fp8 staging registers do not fit).  A
// 64-row unit is held at 2 per SIMD by LDS anyway.
template <int BLK, int KV>
constexpr int waves_per_simd() {
  return (BLK == 128 && KV == BSA_KV_BF16) ? 3 : 2;
}

// KV: BSA_KV_BF16, BSA_KV_FP8E4M3 or BSA_KV_BF16_SCALED (bf16 values with
// per-block scales, folded in exactly as for fp8).  KS: key halves.  With
// KS = 2 two groups of NW waves share the unit: group 0 sweeps the selected
// blocks up to the one where half of the unit's tiles are reached, group 1
// the rest, each on its own pair of LDS stages; the two partial results
// (O, m, l per query row) are merged in a fixed order at the end.  Used for
// short launches, where the heaviest units would otherwise set the time.
template <int BLK, int KV, bool BITMAP, int KS>
__global__ __launch_bounds__(BLK * 2 * KS, (waves_per_simd<BLK, KV>())) void bsa_fwd_kernel(
    FwdParams p) {
  constexpr bool FP8 = KV == BSA_KV_FP8E4M3;  // codes staged through VGPRs
  constexpr bool SCALED = KV != BSA_KV_BF16;  // per-block K/V scales
  constexpr int NW = BLK / 32;  // waves of a key group; each owns 32 query rows
  constexpr int NT = NW * 64;   // threads of a key group
  constexpr int NTA = NT * KS;  // threads of the workgroup
  // Operand reads pinned ahead of their products (K right after the tile is
  // published, V before the softmax) where registers allow: with two waves
  // per SIMD there is room for both operand sets; the block-128 bf16 kernel,
  // capped for three waves per SIMD, leaves the order to the compiler.
  constexpr bool EARLY_OPS = waves_per_simd<BLK, KV>() == 2;
  // All LDS is dynamic, so the stages start at LDS address 0 and every
  // operand address is a per-lane constant plus an immediate offset.
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave_all / NW;      // key group
  const int wave = wave_all % NW;      // wave within the key group
  const int htid = tid - half * NT;    // thread within the key group
  const int g = lane >> 4;    // lane group: 0..3
  const int r16 = lane & 15;  // row within a 16-row MFMA tile

  const int NK = p.NK;
  // LDS: the key groups' stages, then the header (selected blocks, redo
  // flag, split entry, tile counts), the byte map and the block list.
  int* s_hdr = (int*)(smem + KS * NSTAGE * STAGE_BYTES);
  int* s_nsel = s_hdr;
  int* s_redo = s_hdr + 1;
  uint8_t* bmp = (uint8_t*)(smem + KS * NSTAGE * STAGE_BYTES + 32);
  uint32_t* list = (uint32_t*)(bmp + ((NK + 15) & ~15));

  // ---- A1: work unit
  const int u = remap_unit(blockIdx.x, p.n_units);
  const int bh = u / p.NQ;
  // the u-th unit in launch order: q-block order, or the given permutation
  const int qb = p.order ? clampi(p.order[u], 0, p.NQ - 1) : u % p.NQ;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int64_t plane = (int64_t)bh * p.S * HD;  // element offset of Q/O (b, h)
  // query head h reads K/V head h / group (grouped-query attention)
  const int64_t kvh = (int64_t)b * p.Hk + h / p.group;
  const int64_t kvplane = kvh * p.Sk * HD;       // element offset of K/V
  const int64_t row = (int64_t)b * p.meta_sb + (int64_t)h * p.meta_sh + qb;

  const int qrow0 = qb * BLK + wave * 32;  // first query row of this wave

  // ---- A3: Q operands (B operand of S^T = K Q^T): Q[row r16][d kk*32+g*8..],
  // loaded first so that they arrive while the selected set is decoded.
  bf16x8 qreg[2][4];
  {
    const uint16_t* qg = p.q + plane + (int64_t)qrow0 * HD;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qreg[qt][kk] = *(const bf16x8*)(qg + (qt * 16 + r16) * HD + kk * 32 + g * 8);
  }
  if (tid == 0) *s_redo = 0;

  // ---- A2: selected set -> LDS byte map: bmp[kb] = valid keys of kb if
  // selected, else 0 (every thread reads the valid counts of its entries)
  if constexpr (BITMAP) {
    const int8_t* mrow = p.mask + row * NK;
    for (int i = tid; i < NK; i += NTA)
      bmp[i] = mrow[i] != 0 ? (uint8_t)block_valid<BLK>(p.vbs, i) : (uint8_t)0;
  } else {
    for (int i = tid; i < NK; i += NTA) bmp[i] = 0;
    __syncthreads();
    const int n = clampi(p.num[row], 0, p.max_kv);
    const int32_t* irow = p.idx + row * p.max_kv;
    for (int j = tid; j < n; j += NTA) {
      const int kb = irow[j];
      // duplicates store the same value
      if (kb >= 0 && kb < NK) bmp[kb] = (uint8_t)block_valid<BLK>(p.vbs, kb);
    }
  }
  __syncthreads();
  // byte map -> ascending list of selected blocks with >= 1 valid key
  if (wave_all == 0) {
    int base = 0;
    for (int c0 = 0; c0 < NK; c0 += 64) {
      const int kb = c0 + lane;
      const int nv = kb < NK ? (int)bmp[kb] : 0;
      const bool f = nv > 0;
      const uint64_t bal = __ballot(f);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (f) list[pos] = ((uint32_t)kb << 8) | (uint32_t)nv;
      base += __popcll(bal);
    }
    if (lane == 0) *s_nsel = base;
    if constexpr (KS == 2) {
      // Split entry E1: group 0 takes entries [0, E1), where the first half
      // of the unit's tiles ends (at least one entry), group 1 the rest.
      // Tiles of an entry: its valid keys / 32 as a share of the key stream
      // (bf16), or ceil(valid keys / 32) (per-block tiles).
      auto work = [&](int nv) { return SCALED ? (nv + KT - 1) / KT : nv; };
      int total = 0;
      for (int c0 = 0; c0 < base; c0 += 64) {
        int x = c0 + lane < base ? work((int)(list[c0 + lane] & 255u)) : 0;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
        total += x;
      }
      int e1 = base, run = 0, w0 = 0;
      for (int c0 = 0; c0 < base && e1 == base; c0 += 64) {
        const int w = c0 + lane < base ? work((int)(list[c0 + lane] & 255u)) : 0;
        int x = w;  // inclusive scan over the lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(x, o);
          if (lane >= o) x += y;
        }
        // first entry whose inclusive sum reaches half the work
        const uint64_t hit = __ballot(c0 + lane < base && 2 * (run + x) >= total);
        if (hit) {
          const int l0 = __ffsll((unsigned long long)hit) - 1;
          e1 = c0 + l0 + 1;
          w0 = run + __shfl(x, l0);
        }
        run += __shfl(x, 63);
      }
      e1 = min(max(e1, 1), base);
      if (e1 == base) w0 = total;
      if (lane == 0) {
        s_hdr[2] = e1;
        // tiles per group
        s_hdr[3] = SCALED ? w0 : (w0 + KT - 1) / KT;
        s_hdr[4] = SCALED ? total - w0 : (total - w0 + KT - 1) / KT;
      }
    }
  }
  __syncthreads();
  const int nsel = *s_nsel;
  // this key group's entries [e0, e0 + nsel_g) and the steps of the pass
  const int e0 = KS == 2 && half ? s_hdr[2] : 0;
  const int nsel_g = KS == 2 ? (half ? nsel - s_hdr[2] : s_hdr[2]) : nsel;
  const int t_mine = KS == 2 ? (half ? s_hdr[4] : s_hdr[3]) : 0;
  const int t_steps = KS == 2 ? max(s_hdr[3], s_hdr[4]) : 0;

  if (nsel == 0) {
    if (half) return;
    // A8 for a unit with no attended key: exact zeros and the sentinel
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int64_t r = (int64_t)bh * p.S + qrow0 + qt * 16 + r16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(u32x2*)(p.out + r * HD + dt * 16 + g * 4) = u32x2{0u, 0u};
      if (p.lse && g == 0) p.lse[r] = BSA_LSE_EMPTY;
    }
    return;
  }

  constexpr int EB = FP8 ? 1 : 2;  // bytes per K/V element in global memory
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem;
  const char* kplane = (const char*)p.k + kvplane * EB;
  const char* vplane = (const char*)p.v + kvplane * EB;
  const int64_t scale_row = kvh * NK;  // fp8 scales of the K/V head

  // Per-lane constant byte offsets (the XOR swizzles make every address a
  // per-lane base XORed with a constant): K operand kbase ^ (kk << 6),
  // keys 16..31 at +16 rows; V^T transposing reads vbase ^ (dt << 5), rows
  // 16..31 at +16 rows; DMA offsets within a 4-row slice dko / dvo.
  // (the key group's stages start at stage0 bytes)
  const uint32_t stage0 = (uint32_t)(half * NSTAGE * STAGE_BYTES);
  const uint32_t kbase = stage0 + (uint32_t)(r16 * ROWB + ((g ^ r16) << 4));
  const uint32_t vbase = stage0 + (uint32_t)(TILE_BYTES + (lane >> 2) * ROWB +
                                             ((2 * ((lane >> 2) & 7) + ((lane & 3) >> 1)) << 4) +
                                             (lane & 1) * 8);
  const int l4 = lane >> 4, pos = lane & 15;
  // DMA source offsets of this lane for its wave's slices (see issue_bf16).
  // With 4 waves the two slices of a wave share their swizzle, so the
  // stream path keeps one offset per tensor and reaches the second slice
  // 4 KB further through the scalar base (fewer live registers).
  constexpr int KP = (SCALED || NW != 4) ? 8 / NW : 1;
  [[maybe_unused]] uint32_t dko[KP], dvo[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int j = wave + i * NW;
    dko[i] = (uint32_t)(j * 1024 + l4 * ROWB + (((pos ^ l4) ^ ((j & 3) << 2)) << 4));
    dvo[i] = (uint32_t)(j * 1024 + l4 * ROWB + (((pos ^ (2 * l4)) ^ ((j & 1) << 3)) << 4));
  }

  ListCursor cursor{list + e0, nsel_g, 0, 0u, 0u};
  [[maybe_unused]] Fp8Staging<NT> st;
  [[maybe_unused]] float ksc_cur = 1.f, vsc_cur = 1.f, ksc_nxt = 1.f, vsc_nxt = 1.f;

  // Per-block tiles (K/V with per-block scales): starts the loads of tile t
  // into stage `stg` (scaled bf16: DMA; fp8: registers) and fetches the
  // block's scales.
  auto issue = [&](const Tile& t, int stg) {
    const int64_t key0 = (int64_t)t.kb * BLK + t.t0;
    const int nvt = t.nv - t.t0;
    if constexpr (FP8) {
      load_tile_fp8<NT>(st, kplane + key0 * HD, vplane + key0 * HD, nvt, htid);
    } else if constexpr (SCALED) {
      const char* kg = kplane + key0 * ROWB;
      const char* vg = vplane + key0 * ROWB;
      const uint32_t sl = smem_lds + stage0 + stg * STAGE_BYTES;
      issue_bf16<NW>(kg, vg, sl, sl + TILE_BYTES, dko, dvo, wave, l4, nvt);
    }
    if constexpr (SCALED) {
      ksc_nxt = p.k_scale[scale_row + t.kb];
      vsc_nxt = p.v_scale[scale_row + t.kb];
    }
  };

  // bf16 K/V without scales: the valid keys of the selected blocks, in
  // list order, form one stream that is cut into 32-row tiles, so a tile
  // may span several blocks and only the unit's last tile is partial.
  // Starts the loads of the tile that begins at stream position w into
  // stage `stg`, moves w past it and returns the tile's row count (1..32).
  // A tile inside one block loads like a block tile; a tile that spans
  // blocks adds, per lane, the offset of the run of rows its row falls in.
  // Rows past the count re-read row 0's chunk.
  auto issue_stream = [&](Walk& w, int stg) -> int {
    const uint32_t sl = smem_lds + stage0 + stg * STAGE_BYTES;
    return next_stream_tile<BLK, NW>(
        cursor, w, nsel_g, wave, l4, lane,
        [&](int64_t key0) {
          const char* kg = kplane + key0 * ROWB;
          const char* vg = vplane + key0 * ROWB;
#pragma unroll
          for (int i = 0; i < 8 / NW; ++i) {
            const uint32_t j = (uint32_t)(wave + i * NW);
            const int xb = (i / KP) * KP * NW * 1024;  // slice bytes past dko
            dma16(kg + xb, dko[i % KP], sl + j * 1024u);
            dma16(vg + xb, dvo[i % KP], sl + TILE_BYTES + j * 1024u);
          }
        },
        [&](int64_t key0, int rows, const uint32_t (&ex)[8 / NW]) {
          const char* kg = kplane + key0 * ROWB;
          const char* vg = vplane + key0 * ROWB;
#pragma unroll
          for (int i = 0; i < 8 / NW; ++i) {
            const int j = wave + i * NW;
            const bool ok = 4 * j + l4 < rows;
            const uint32_t xb = (uint32_t)((i / KP) * KP * NW * 1024);
            const uint32_t ko = dko[i % KP], vo = dvo[i % KP];
            dma16(kg, ok ? ko + xb + ex[i] : (ko & 0xFFu), sl + (uint32_t)j * 1024u);
            dma16(vg, ok ? vo + xb + ex[i] : (vo & 0xFFu),
                  sl + TILE_BYTES + (uint32_t)j * 1024u);
          }
        });
  };

  // One pass of the K loop over every selected tile.
  //  SAFE = false: the reference m of each row is fixed at the first tile's
  //  row maximum; weights 2^(t - m) may exceed 1 but the accumulators are
  //  never rescaled.  The caller checks afterwards that nothing overflowed.
  //  SAFE = true: online softmax -- every tile raises m to the running
  //  maximum and rescales O and l by 2^(m_old - m_new).
  // Both give the same O and LSE in exact arithmetic (any reference does).
  auto run_pass = [&](auto safe_c, Acc& acc) {
    constexpr bool SAFE = decltype(safe_c)::value;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) acc.o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m[0] = acc.m[1] = -INFINITY;
    acc.l[0] = acc.l[1] = 0.f;

    cursor.reset(lane);
    [[maybe_unused]] Tile cur{};
    [[maybe_unused]] Walk walk{0, 0};
    [[maybe_unused]] int cur_rows = 0;
    if (nsel_g > 0) {
      if constexpr (SCALED) {
        cur = cursor.at(0, lane);
        issue(cur, 0);
      } else {
        cur_rows = issue_stream(walk, 0);
      }
      if constexpr (FP8) store_tile_fp8<NT>(st, smem + stage0, htid);
      if constexpr (SCALED) {
        ksc_cur = ksc_nxt;
        vsc_cur = vsc_nxt;
      }
    }

    // stg_c: LDS stage of `cur` (compile-time); first_c: this is tile 0
    // (active = false: this key group has no tile left; it only takes part
    // in the workgroup's barrier)
    auto step = [&](auto stg_c, auto first_c, bool active) -> bool {
      constexpr int STG = decltype(stg_c)::value;
      constexpr bool FIRST = decltype(first_c)::value != 0;
      // tile `cur` complete in LDS for every wave; stage STG^1 free again
      wait_vm_all();
      __syncthreads();
      if (!active) return true;
      const char* sb = smem + STG * STAGE_BYTES;
      [[maybe_unused]] Tile nxt{};
      [[maybe_unused]] int nxt_rows = 0;
      bool has_next = false;
      // Loads of the next tile.  fp8 tiles come through registers and are
      // stored to LDS at the end of this step, so their loads go out first;
      // DMA tiles have a whole step of slack, so the K operand reads of this
      // tile go out first.
      auto issue_next = [&]() {
        if constexpr (SCALED) {
          nxt = cursor.next(cur, lane);
          has_next = nxt.e < nsel_g;
          if (has_next) issue(nxt, STG ^ 1);
        } else {
          has_next = walk.e < nsel_g;
          if (has_next) nxt_rows = issue_stream(walk, STG ^ 1);
        }
      };
      if constexpr (FP8) issue_next();
      KOps ko;
      if constexpr (EARLY_OPS) {
        load_k(sb, kbase, ko);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!FP8) issue_next();
      int nvt;  // valid keys of this tile (>= 1)
      if constexpr (SCALED) nvt = cur.nv - cur.t0;
      else nvt = cur_rows;
      const int lim = nvt - 4 * g;
      float cs = p.c;
      float vsc = 1.f;
      if constexpr (SCALED) {
        cs *= ksc_cur;
        vsc = vsc_cur;
      }

      // ---- A5 + A6: scores, the reference update (first tile, or every
      // tile of the rescaling pass) and the exponents in t-space.  The two
      // tile kinds differ up to here only; the paths join before the V reads
      // are issued.
      float sv[2][8];
      auto scores = [&](auto kind_c) {
        constexpr int KIND = decltype(kind_c)::value;
        if constexpr (!EARLY_OPS) load_k(sb, kbase, ko);
        tile_scores<KIND>(ko, qreg, nvt, sv);
        if constexpr (SAFE || FIRST) {
          float tm[2];
          tile_max<KIND>(sv, cs, lim, tm);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const float mnew = fmaxf(acc.m[qt], tm[qt]);
            if constexpr (SAFE && !FIRST) {
              const float alpha = __builtin_amdgcn_exp2f(acc.m[qt] - mnew);
              acc.l[qt] *= alpha;
#pragma unroll
              for (int dt = 0; dt < 8; ++dt) acc.o[dt][qt] *= alpha;
            }
            acc.m[qt] = mnew;
          }
        }
        tile_exponents<KIND>(sv, cs, lim, acc);
      };
      if (nvt >= KT) scores(IntC<FULL>{});
      else scores(IntC<PART>{});
      VOps vo;
      if constexpr (EARLY_OPS) {
        load_v(sb, vbase, vo);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 pop[2];
      tile_probs<SCALED>(sv, vsc, acc, pop);

      // ---- A7: PV
      if constexpr (!EARLY_OPS) load_v(sb, vbase, vo);
      tile_pv(vo, pop, acc);

      if (!has_next) return true;
      if constexpr (FP8) store_tile_fp8<NT>(st, smem + stage0 + (STG ^ 1) * STAGE_BYTES, htid);
      if constexpr (SCALED) {
        ksc_cur = ksc_nxt;
        vsc_cur = vsc_nxt;
        cur = nxt;
      } else {
        cur_rows = nxt_rows;
      }
      return false;
    };

    if constexpr (KS == 1) {
      if (!step(IntC<0>{}, IntC<1>{}, true)) {
        while (true) {
          if (step(IntC<1>{}, IntC<0>{}, true)) break;
          if (step(IntC<0>{}, IntC<0>{}, true)) break;
        }
      }
    } else {
      // both key groups take t_steps barrier steps; a group whose tiles are
      // done idles through the rest
      int s = 0;
      step(IntC<0>{}, IntC<1>{}, s < t_mine);
      for (++s; s < t_steps; ++s) {
        step(IntC<1>{}, IntC<0>{}, s < t_mine);
        if (++s >= t_steps) break;
        step(IntC<0>{}, IntC<0>{}, s < t_mine);
      }
    }
  };

  // The fixed-reference pass is valid for any sign of the score scale (the
  // first tile's maximum is taken over t = s*cs) unless a weight or a sum
  // overflowed: a score more than ~2^7 log2 units above the first tile's
  // maximum.  Then the unit is recomputed with the online rescale.
  Acc acc;
  run_pass(IntC<0>{}, acc);
  bool bad = !(acc.l[0] <= 1e37f) || !(acc.l[1] <= 1e37f);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bad |= !(__builtin_fabsf(acc.o[dt][qt][i]) <= 3e38f);
  if (__any(bad)) *s_redo = 1;
  __syncthreads();  // every wave is done with both stages; s_redo visible
  if (*s_redo) run_pass(IntC<1>{}, acc);

  if constexpr (KS == 2) {
    // Merge of the key groups' partial results for the same query rows:
    // group 1 hands O, m and l over through LDS, group 0 combines
    //   m = max(m0, m1) + 1,  O = O0 2^(m0-m) + O1 2^(m1-m),  l likewise
    // (a group without tiles has m = -inf, O = l = 0 and weighs 0).  The
    // + 1 halves both weights, exactly, so that the sum of two partial O
    // that each passed the overflow check stays finite; O/l and m + log2 l
    // are unchanged by it.
    float* mb = (float*)smem;  // [68][NW][64], after every wave left its stages
    auto at = [&](int i) -> float& { return mb[(i * NW + wave) * 64 + lane]; };
    __syncthreads();
    if (half) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i) at((dt * 2 + qt) * 4 + i) = acc.o[dt][qt][i];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        at(64 + qt) = acc.m[qt];
        at(66 + qt) = acc.l[qt];
      }
    }
    __syncthreads();
    if (half) return;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float m1 = at(64 + qt);
      const float m = fmaxf(acc.m[qt], m1) + 1.f;
      const float a0 = __builtin_amdgcn_exp2f(acc.m[qt] - m);
      const float a1 = __builtin_amdgcn_exp2f(m1 - m);
      acc.l[qt] = acc.l[qt] * a0 + at(66 + qt) * a1;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc.o[dt][qt][i] = acc.o[dt][qt][i] * a0 + at((dt * 2 + qt) * 4 + i) * a1;
      acc.m[qt] = m;
    }
  }

  // ---- A8: epilogue
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    // >= 1 (>= 1/2 after a merge): the reference key has weight >= 1
    const float l = group_sum(acc.l[qt]);
    const float inv = 1.0f / l;
    const int64_t r = (int64_t)bh * p.S + qrow0 + qt * 16 + r16;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o = acc.o[dt][qt] * inv;
      *(u32x2*)(p.out + r * HD + dt * 16 + g * 4) =
          u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    if (p.lse && g == 0) p.lse[r] = acc.m[qt] + __builtin_amdgcn_logf(l);
  }
}

// ----------------------------------------------------------------------------
// host side

size_t lds_bytes(int NK, int KS) {
  return (size_t)KS * NSTAGE * STAGE_BYTES + 32 + (size_t)((NK + 15) & ~15) +
         (size_t)NK * sizeof(uint32_t);
}

template <int BLK, int KV, bool BITMAP, int KS>
bsa_status launch(const FwdParams& p, hipStream_t stream) {
  auto kern = bsa_fwd_kernel<BLK, KV, BITMAP, KS>;
  const size_t lds = lds_bytes(p.NK, KS);
  if (lds > 65536) {
    if (hipFuncSetAttribute((const void*)kern,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
  }
  hipLaunchKernelGGL(kern, dim3(p.n_units), dim3(BLK * 2 * KS), lds, stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <bool BITMAP, int BLK>
bsa_status dispatch_kv(const FwdParams& p, int kv, hipStream_t s) {
  switch (kv) {
    case BSA_KV_FP8E4M3: return launch<BLK, BSA_KV_FP8E4M3, BITMAP, 1>(p, s);
    case BSA_KV_BF16_SCALED: return launch<BLK, BSA_KV_BF16_SCALED, BITMAP, 1>(p, s);
    default:
      // short launches split each unit's keys over two wave groups (with
      // more units than run at once, whole units balance better)
      if constexpr (BLK == 64)
        if (p.n_units <= BSA_FWD_KEY_SPLIT_MAX_UNITS)
          return launch<BLK, BSA_KV_BF16, BITMAP, 2>(p, s);
      return launch<BLK, BSA_KV_BF16, BITMAP, 1>(p, s);
  }
}

template <bool BITMAP>
bsa_status dispatch(const FwdParams& p, int block, int kv, hipStream_t s) {
  if (block == 64) return dispatch_kv<BITMAP, 64>(p, kv, s);
  return dispatch_kv<BITMAP, 128>(p, kv, s);
}

bool aligned16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

// Static checks shared by both forms.
bsa_status check_common(const void* q, const void* k, const void* v,
                        int32_t kv_dtype, const float* k_scale,
                        const float* v_scale, const void* out, int32_t B,
                        int32_t H, int32_t Hk, int32_t S, int32_t Sk,
                        int32_t D, int32_t block) {
  if (!q || !k || !v || !out) return BSA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hk <= 0 || S <= 0 || Sk <= 0 || D <= 0 || block <= 0)
    return BSA_ERR_SHAPE;
  if (S % block != 0 || Sk % block != 0 || H % Hk != 0) return BSA_ERR_SHAPE;
  if (D != HD) return BSA_ERR_UNSUPPORTED;
  if (block != 64 && block != 128) return BSA_ERR_UNSUPPORTED;
  if (kv_dtype != BSA_KV_BF16 && kv_dtype != BSA_KV_FP8E4M3 &&
      kv_dtype != BSA_KV_BF16_SCALED)
    return BSA_ERR_UNSUPPORTED;
  if (kv_dtype != BSA_KV_BF16 && (!k_scale || !v_scale)) return BSA_ERR_NULL;
  if (Sk / block > BSA_MAX_KEY_BLOCKS) return BSA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)B * H * (S / block);
  if (units > INT32_MAX || (int64_t)B * H * S > INT32_MAX ||
      (int64_t)B * Hk * Sk > INT32_MAX)
    return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return BSA_ERR_ALIGN;
  return BSA_OK;
}

// sm_scale: any finite value (zero and negative included).
bool finite_scale(float x) { return __builtin_isfinite(x); }

FwdParams make_params(const void* q, const void* k, const void* v,
                      const float* k_scale, const float* v_scale,
                      const int32_t* vbs, float sm_scale, void* out, float* lse,
                      int32_t B, int32_t H, int32_t Hk, int32_t S, int32_t Sk,
                      int32_t block) {
  FwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = k;
  p.v = v;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.vbs = vbs;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.c = sm_scale * LOG2E;
  p.H = H;
  p.Hk = Hk;
  p.group = H / Hk;
  p.S = S;
  p.Sk = Sk;
  p.NQ = S / block;
  p.NK = Sk / block;
  p.n_units = B * H * (S / block);
  return p;
}

}  // namespace

extern "C" bsa_status bsa_fwd_lut_ordered(
    const void* q, const void* k, const void* v, int32_t kv_dtype,
    const float* k_scale, const float* v_scale, const int32_t* q2k_idx,
    const int32_t* q2k_num, int32_t max_kv, int64_t meta_stride_b,
    int64_t meta_stride_h, const int32_t* variable_block_sizes,
    const int32_t* qblock_order, float sm_scale, void* out, float* lse, int32_t B,
    int32_t H, int32_t Hk, int32_t S, int32_t Sk, int32_t D, int32_t block,
    void* stream) {
  bsa_status st = check_common(q, k, v, kv_dtype, k_scale, v_scale, out, B, H,
                               Hk, S, Sk, D, block);
  if (st != BSA_OK) return st;
  if (!finite_scale(sm_scale)) return BSA_ERR_VALUE;
  if (!q2k_idx || !q2k_num) return BSA_ERR_NULL;
  if (max_kv < 1 || meta_stride_b < 0 || meta_stride_h < 0) return BSA_ERR_SHAPE;
  FwdParams p = make_params(q, k, v, k_scale, v_scale, variable_block_sizes,
                            sm_scale, out, lse, B, H, Hk, S, Sk, block);
  p.idx = q2k_idx;
  p.num = q2k_num;
  p.order = qblock_order;
  p.max_kv = max_kv;
  p.meta_sb = meta_stride_b;
  p.meta_sh = meta_stride_h;
  return dispatch<false>(p, block, kv_dtype,
                         (hipStream_t)stream);
}

extern "C" bsa_status bsa_fwd_lut(const void* q, const void* k, const void* v,
                                  int32_t kv_dtype, const float* k_scale,
                                  const float* v_scale, const int32_t* q2k_idx,
                                  const int32_t* q2k_num, int32_t max_kv,
                                  int64_t meta_stride_b, int64_t meta_stride_h,
                                  const int32_t* variable_block_sizes,
                                  float sm_scale, void* out, float* lse,
                                  int32_t B, int32_t H, int32_t Hk, int32_t S,
                                  int32_t Sk, int32_t D, int32_t block,
                                  void* stream) {
  return bsa_fwd_lut_ordered(q, k, v, kv_dtype, k_scale, v_scale, q2k_idx, q2k_num,
                             max_kv, meta_stride_b, meta_stride_h,
                             variable_block_sizes, nullptr, sm_scale, out, lse, B, H,
                             Hk, S, Sk, D, block, stream);
}

extern "C" bsa_status bsa_fwd_bitmap_ordered(
    const void* q, const void* k, const void* v, int32_t kv_dtype,
    const float* k_scale, const float* v_scale, const int8_t* mask,
    int64_t mask_stride_b, int64_t mask_stride_h,
    const int32_t* variable_block_sizes, const int32_t* qblock_order,
    float sm_scale, void* out, float* lse, int32_t B, int32_t H, int32_t Hk,
    int32_t S, int32_t Sk, int32_t D, int32_t block, void* stream) {
  bsa_status st = check_common(q, k, v, kv_dtype, k_scale, v_scale, out, B, H,
                               Hk, S, Sk, D, block);
  if (st != BSA_OK) return st;
  if (!finite_scale(sm_scale)) return BSA_ERR_VALUE;
  if (!mask) return BSA_ERR_NULL;
  if (mask_stride_b < 0 || mask_stride_h < 0) return BSA_ERR_SHAPE;
  FwdParams p = make_params(q, k, v, k_scale, v_scale, variable_block_sizes,
                            sm_scale, out, lse, B, H, Hk, S, Sk, block);
  p.mask = mask;
  p.order = qblock_order;
  p.meta_sb = mask_stride_b;
  p.meta_sh = mask_stride_h;
  return dispatch<true>(p, block, kv_dtype,
                        (hipStream_t)stream);
}

extern "C" bsa_status bsa_fwd_bitmap(const void* q, const void* k, const void* v,
                                     int32_t kv_dtype, const float* k_scale,
                                     const float* v_scale, const int8_t* mask,
                                     int64_t mask_stride_b, int64_t mask_stride_h,
                                     const int32_t* variable_block_sizes,
                                     float sm_scale, void* out, float* lse,
                                     int32_t B, int32_t H, int32_t Hk,
                                     int32_t S, int32_t Sk, int32_t D,
                                     int32_t block, void* stream) {
  return bsa_fwd_bitmap_ordered(q, k, v, kv_dtype, k_scale, v_scale, mask,
                                mask_stride_b, mask_stride_h, variable_block_sizes,
                                nullptr, sm_scale, out, lse, B, H, Hk, S, Sk, D,
                                block, stream);
}

extern "C" const char* bsa_status_str(int32_t status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_NULL: return "a required pointer is NULL";
    case BSA_ERR_SHAPE:
      return "invalid size (<= 0, S or Sk not a multiple of block, or H not a "
             "multiple of Hk)";
    case BSA_ERR_UNSUPPORTED:
      return "unsupported configuration (D != 128, block not 64/128, "
             "too many key blocks, or unknown kv dtype)";
    case BSA_ERR_ALIGN: return "q, k, v or out is not 16-byte aligned";
    case BSA_ERR_HIP: return "HIP launch error";
    case BSA_ERR_VALUE: return "sm_scale is not finite";
    default: return "unknown status";
  }
}
