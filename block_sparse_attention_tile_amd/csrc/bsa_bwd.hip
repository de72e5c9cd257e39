// bsa_bwd.hip -- gradients of the block-sparse attention forward pass on
// MI355X (gfx950).
//
// The forward pass returns O and the base-2 row LSE so that a backward pass
// can rebuild the softmax weights without a second reduction (FastVideo
// "block_sparse_attn_sm100a.py": the LSE-producing path is kept for
// forward/backward pairing).  With t = (q . k) * sm_scale * log2(e):
//
//   P  = 2^(t - LSE)                (the forward weights, normalised)
//   dP = dO V^T,   delta = rowsum(dO * O),   dS = P * (dP - delta)
//   dQ = sm_scale * dS K,  dK = sm_scale * dS^T Q,  dV = P^T dO
//
// over each unit's attended keys.  Four launches:
//   1. delta_kernel     delta[row] = sum_d O * dO (fp32), one pass over O, dO.
//   2. k2q_kernel       the transposed selection: for every (b, K/V head,
//                       key block) a byte per (query head of the group,
//                       query block) that attends it (1 = attends, the key
//                       block has >= 1 valid key).  Duplicate stores write
//                       the same 1, so no atomics are needed.
//   3. dq_kernel        one workgroup per query unit, the same walk as the
//                       forward pass (32-row tiles cut from the stream of
//                       the unit's valid keys); dQ accumulates in registers
//                       and is written once.
//   4. dkdv_kernel      one workgroup per (b, K/V head, key block), launched
//                       heaviest first per K/V head (kunit_work_kernel and
//                       the rank pass order them; dq_kernel's units are
//                       ordered likewise with the LUT form): its keys
//                       stay in registers while it walks every query unit
//                       that attends the block (from the byte map), so dK and
//                       dV are complete in one workgroup -- grouped query
//                       heads included -- and written once, without atomics.
//
// All MFMA work is v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation); P and dS are rounded to bf16 as operands, the outputs to
// bf16 (RNE).

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "bsa.h"
#include "bsa_device.h"

// launch-order ranking of work values, in bsa_order.hip
bsa_status bsa_rank_runs(int32_t* order, int32_t groups, int32_t n, hipStream_t stream);

namespace {

constexpr int BSTAGE = 2 * TILE_BYTES;  // two 32-row tiles per stage
// A launch of at most this many workgroups runs them all at once (256 CUs
// hold up to 4 each), so it is not reordered.
constexpr int64_t ORDER_MIN_UNITS = 1024;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  const int32_t* idx;   // LUT form
  const int32_t* num;
  const int8_t* mask;   // bitmap form
  const int8_t* k2q;    // [B*Hk*NK, G*NQ]
  const int32_t* order; // LUT form: q-block launch order of dq per (b, h), or null
  const int32_t* korder; // key-block launch order of dk/dv per (b, K/V head), or null
  int64_t meta_sb, meta_sh;
  const int32_t* vbs;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float c;              // sm_scale * log2(e)
  float sm_scale;
  int32_t max_kv;
  int32_t H, Hk, group, S, Sk, NQ, NK;
  int32_t n_units;
};

// ---------------------------------------------------------------------------
// 1. delta = rowsum(O * dO): 16 lanes per 128-element row, 16 B per lane.

__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    float* __restrict__ delta,
                                                    int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(out + row * HD + part * 8);
    const u32x4 b = *(const u32x4*)(dout + row * HD + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
      s += __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(b[i] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
  if (row < rows && part == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------
// 2. transposed selection map.

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* __restrict__ p,
                                                        int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{0, 0, 0, 0};
}

__global__ __launch_bounds__(256) void fill_zero_bytes_kernel(int8_t* __restrict__ p,
                                                              int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// One wave per query unit (b, h, qb): every selected key block kb with at
// least one valid key sets byte [(b*Hk + h/G)*NK + kb][(h%G)*NQ + qb].
template <bool BITMAP>
__global__ __launch_bounds__(256) void k2q_kernel(BwdParams p) {
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (u >= p.n_units) return;
  const int qb = (int)(u % p.NQ);
  const int64_t bh = u / p.NQ;
  const int h = (int)(bh % p.H);
  const int b = (int)(bh / p.H);
  const int64_t row = (int64_t)b * p.meta_sb + (int64_t)h * p.meta_sh + qb;
  const int64_t gq = (int64_t)p.group * p.NQ;
  int8_t* base = (int8_t*)p.k2q + ((int64_t)b * p.Hk + h / p.group) * p.NK * gq +
                 (int64_t)(h % p.group) * p.NQ + qb;
  if constexpr (BITMAP) {
    const int8_t* mrow = p.mask + row * p.NK;
    for (int kb = lane; kb < p.NK; kb += 64)
      if (mrow[kb] != 0 && (p.vbs == nullptr || p.vbs[kb] > 0)) base[kb * gq] = 1;
  } else {
    const int n = clampi(p.num[row], 0, p.max_kv);
    const int32_t* irow = p.idx + row * p.max_kv;
    for (int j = lane; j < n; j += 64) {
      const int kb = irow[j];
      if (kb >= 0 && kb < p.NK && (p.vbs == nullptr || p.vbs[kb] > 0))
        base[(int64_t)kb * gq] = 1;
    }
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two gradient kernels.

// dK/dV launch order, pass 1: the work of key-block unit u = (b*Hk + kvh)*NK
// + kb is the number of query units set in its map row (0 for a block with
// no valid key); bsa_rank_runs then orders each (b, K/V head) heaviest
// first.  One wave per unit.
__global__ __launch_bounds__(256) void kunit_work_kernel(BwdParams p, int32_t* work,
                                                         int32_t n_kunits) {
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (u >= n_kunits) return;
  const int kb = (int)(u % p.NK);
  const int64_t gq = (int64_t)p.group * p.NQ;
  const uint8_t* row = (const uint8_t*)p.k2q + u * gq;
  int c = 0;
  if (!p.vbs || p.vbs[kb] > 0) {
    if ((gq & 3) == 0) {  // rows 4-byte aligned: the map starts 256-aligned
      const uint32_t* w4 = (const uint32_t*)row;
      for (int64_t i = lane; i < gq / 4; i += 64) {
        const uint32_t x = w4[i];
        c += ((x & 0xFFu) != 0) + ((x & 0xFF00u) != 0) + ((x & 0xFF0000u) != 0) +
             ((x & 0xFF000000u) != 0);
      }
    } else {
      for (int64_t i = lane; i < gq; i += 64) c += row[i] != 0;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) work[u] = c;
}

// Ascending list of the set entries of an LDS byte map of n entries, each
// entry stored as (index << 8) | payload, payload = map byte.  One wave.
__device__ __forceinline__ int compact_list(const uint8_t* map, int n,
                                            uint32_t* list, int lane) {
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int i = c0 + lane;
    const uint32_t m = i < n ? map[i] : 0u;
    const bool f = m != 0;
    const uint64_t bal = __ballot(f);
    const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
    if (f) list[pos] = ((uint32_t)i << 8) | m;
    base += __popcll(bal);
  }
  return base;
}

// Tiles of the backward kernels are read both row-wise (MFMA A operands: 16
// rows x one 16-byte chunk per 16 lanes) and through the transposing read
// (8 rows x two chunks per 32 lanes).  Chunk c of row r sits at position
// c ^ bswz(r) with bswz(r) = (r ^ 2r) mod 16: a permutation of the 16 rows
// (row reads hit 16 distinct positions) whose values shifted right by one
// are distinct within each group of 8 rows (transposing reads hit 16
// distinct positions), so both are free of bank conflicts.  (The row
// swizzle c ^ r of the forward's K tiles costs the transposing read a
// 2-way conflict.)
__device__ __forceinline__ int bswz(int r) { return (r ^ (r << 1)) & 15; }

// Address of this lane's transposing read (ds_read_b64_tr_b16) of a tile:
// rows lane/4 (and +16), the 4-element column group (lane & 3) of 16-column
// group dt: base ^ (dt << 5).
__device__ __forceinline__ uint32_t tr_base(int lane) {
  const int row = lane >> 2;
  const int hb = (lane & 3) >> 1;
  return (uint32_t)(row * ROWB + ((hb ^ bswz(row)) << 4) + (lane & 1) * 8);
}

__device__ __forceinline__ bf16x8 tr_read(const char* tile, uint32_t addr) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + addr));
  const i16x4 b =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + addr + 16 * ROWB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  const u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                    pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, pk);
}

// ---------------------------------------------------------------------------
// 3. dQ: one workgroup per query unit, BLK/32 waves of 32 query rows.
//
// Per 32-key tile (K and V tiles in LDS, both stored with bswz):
//   S^T[key][q] = K Q^T              A = K rows,   B = Q (registers)
//   P^T = 2^(S^T c - LSE_q)          keys past the block's count -> 0
//   dP^T[key][q] = V dO^T            A = V rows,   B = dO (registers)
//   dS^T = P^T (dP^T - delta_q)
//   dQ^T[d][q] += K^T dS^T           A = K^T (transposing reads), B = dS^T
// The accumulator layout of dS^T is the B operand layout with the key
// permutation 8g+i <-> 4g+i / 16+4g+(i-4), matched by the transposing reads
// of rows lane/4 and lane/4 + 16.

template <int BLK, bool BITMAP>
__global__ __launch_bounds__(BLK * 2, 2) void dq_kernel(BwdParams p) {
  constexpr int NW = BLK / 32;
  constexpr int NT = NW * 64;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int NK = p.NK;
  int* s_nsel = (int*)(smem + 2 * BSTAGE);
  uint8_t* bmp = (uint8_t*)(smem + 2 * BSTAGE + 16);
  uint32_t* list = (uint32_t*)(bmp + ((NK + 15) & ~15));

  const int u = remap_unit(blockIdx.x, p.n_units);
  const int bh = u / p.NQ;
  // the u-th unit in launch order (heaviest first with the LUT form)
  const int qb = p.order ? clampi(p.order[u], 0, p.NQ - 1) : u % p.NQ;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int64_t plane = (int64_t)bh * p.S * HD;
  const int64_t kvh = (int64_t)b * p.Hk + h / p.group;
  const int64_t kvplane = kvh * p.Sk * HD;
  const int64_t row = (int64_t)b * p.meta_sb + (int64_t)h * p.meta_sh + qb;
  const int qrow0 = qb * BLK + wave * 32;

  // Q and dO as B operands: row r16 (+16 qt), columns kk*32 + g*8 ..; loaded
  // first so that they arrive while the selected set is decoded.
  bf16x8 qreg[2][4], doreg[2][4];
  float lse[2], dlt[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int64_t r = (int64_t)bh * p.S + qrow0 + qt * 16 + r16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qreg[qt][kk] = *(const bf16x8*)(p.q + r * HD + kk * 32 + g * 8);
      doreg[qt][kk] = *(const bf16x8*)(p.dout + r * HD + kk * 32 + g * 8);
    }
    lse[qt] = p.lse[r];
    dlt[qt] = p.delta[r];
  }

  // selected set -> bmp[kb] = valid keys of kb if selected, else 0
  if constexpr (BITMAP) {
    const int8_t* mrow = p.mask + row * NK;
    for (int i = tid; i < NK; i += NT)
      bmp[i] = mrow[i] != 0 ? (uint8_t)block_valid<BLK>(p.vbs, i) : 0;
  } else {
    for (int i = tid; i < NK; i += NT) bmp[i] = 0;
    __syncthreads();
    const int n = clampi(p.num[row], 0, p.max_kv);
    const int32_t* irow = p.idx + row * p.max_kv;
    for (int j = tid; j < n; j += NT) {
      const int kb = irow[j];
      if (kb >= 0 && kb < NK) bmp[kb] = (uint8_t)block_valid<BLK>(p.vbs, kb);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int n = compact_list(bmp, NK, list, lane);
    if (lane == 0) *s_nsel = n;
  }
  __syncthreads();
  const int nsel = *s_nsel;

  if (nsel == 0) {  // no attended key: dQ = 0
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int64_t r = (int64_t)bh * p.S + qrow0 + qt * 16 + r16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *(u32x2*)(p.dq + r * HD + dt * 16 + g * 4) = u32x2{0u, 0u};
    }
    return;
  }

  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem;
  const char* kplane = (const char*)(p.k + kvplane);
  const char* vplane = (const char*)(p.v + kvplane);

  const int l4 = lane >> 4, pos = lane & 15;
  uint32_t dko[8 / NW];
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) {
    const int j = wave + i * NW;
    dko[i] = (uint32_t)(j * 1024 + l4 * ROWB + ((pos ^ bswz(4 * j + l4)) << 4));
  }
  const uint32_t kbase = (uint32_t)(r16 * ROWB + ((g ^ bswz(r16)) << 4));
  const uint32_t trb = tr_base(lane);

  f32x4 acc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    acc[dt][0] = acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles are cut from the stream of the unit's valid keys (a tile may
  // span blocks; only the last one is partial).
  ListCursor cursor{list, nsel, 0, 0u, 0u};
  cursor.reset(lane);
  Walk walk{0, 0};
  auto issue = [&](int stg) -> int {
    const uint32_t sl = smem_lds + stg * BSTAGE;
    return next_stream_tile<BLK, NW>(
        cursor, walk, nsel, wave, l4, lane,
        [&](int64_t key0) {
          issue_rows<NW>(kplane + key0 * ROWB, sl, dko, wave, l4, KT);
          issue_rows<NW>(vplane + key0 * ROWB, sl + TILE_BYTES, dko, wave, l4, KT);
        },
        [&](int64_t key0, int rows, const uint32_t (&ex)[8 / NW]) {
          issue_split_rows<NW>(kplane + key0 * ROWB, sl, dko, ex, rows, wave, l4);
          issue_split_rows<NW>(vplane + key0 * ROWB, sl + TILE_BYTES, dko, ex, rows, wave,
                               l4);
        });
  };

  int cur_rows = issue(0);
  auto step = [&](auto stg_c) -> bool {
    constexpr int STG = decltype(stg_c)::value;
    wait_vm_all();
    __syncthreads();
    const bool has_next = walk.e < nsel;
    const int nxt_rows = has_next ? issue(STG ^ 1) : 0;
    const int lim = cur_rows - 4 * g;  // valid keys of this lane's group
    const char* kt = smem + STG * BSTAGE;
    const char* vt = kt + TILE_BYTES;

    // S^T and dP^T, both 2 key halves x 2 query tiles
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t a = (kbase ^ (kk << 6)) + hh * 16 * ROWB;
        const bf16x8 kop = *(const bf16x8*)(kt + a);
        const bf16x8 vop = *(const bf16x8*)(vt + a);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          s[hh][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kop, qreg[qt][kk], kk == 0 ? z : s[hh][qt], 0, 0, 0);
          dp[hh][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              vop, doreg[qt][kk], kk == 0 ? z : dp[hh][qt], 0, 0, 0);
        }
      }
    // dS^T, packed as B operands (8 keys per lane: 4 of each half)
    bf16x8 dsop[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int hh = e >> 2, j = e & 3;
        const float pr = 16 * hh + j < lim
                             ? __builtin_amdgcn_exp2f(
                                   __builtin_fmaf(s[hh][qt][j], p.c, -lse[qt]))
                             : 0.f;
        x[e] = pr * (dp[hh][qt][j] - dlt[qt]);
      }
      dsop[qt] = pack8(x);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x8 ktop = tr_read(kt, trb ^ (uint32_t)(dt << 5));
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ktop, dsop[qt],
                                                               acc[dt][qt], 0, 0, 0);
    }
    if (!has_next) return true;
    cur_rows = nxt_rows;
    return false;
  };
  while (true) {
    if (step(IntC<0>{})) break;
    if (step(IntC<1>{})) break;
  }

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int64_t r = (int64_t)bh * p.S + qrow0 + qt * 16 + r16;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o = acc[dt][qt] * p.sm_scale;
      *(u32x2*)(p.dq + r * HD + dt * 16 + g * 4) =
          u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

// ---------------------------------------------------------------------------
// 4. dK, dV: one workgroup per (b, K/V head, key block), BLK/16 waves of 16
// keys each (blocks with at most BLK/2 valid keys: two waves per 16 keys,
// each on half the query rows).  The keys' K and V rows are B operands in registers (rows past
// the block's valid count zeroed).  For every attending query unit, in
// 64-row query steps (Q and dO as two 32-row tiles each in LDS with the row
// swizzle bswz, the rows' LSE and delta beside them):
//   S[q][key] = Q K^T                A = Q rows,   B = K^T (registers)
//   P = 2^(S c - LSE_q),  0 for keys past the count
//   dP[q][key] = dO V^T              A = dO rows,  B = V^T (registers)
//   dS = P (dP - delta_q)
//   dV^T[d][key] += dO^T P           A = dO^T (transposing reads), B = P
//   dK^T[d][key] += Q^T dS           A = Q^T (transposing reads),  B = dS
// P and dS are B operands with the query permutation 8g+i <-> 4g+i /
// 16+4g+(i-4) across two 16-row query sub-tiles.

constexpr int QSTEP = 64;                                 // query rows per step
constexpr int DSTAGE = 4 * TILE_BYTES + 1024;             // Q, dO, LSE, delta
constexpr int LSE_OFF = 4 * TILE_BYTES;                   // 64 floats
constexpr int DLT_OFF = 4 * TILE_BYTES + 256;             // 64 floats

template <int BLK>
__global__ __launch_bounds__(BLK * 4, 2) void dkdv_kernel(BwdParams p) {
  constexpr int NW = BLK / 16;
  constexpr int NT = NW * 64;
  constexpr int QT_PER_UNIT = BLK / QSTEP;  // query steps per unit
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int gq = p.group * p.NQ;  // map entries per key block
  int* s_n = (int*)(smem + 2 * DSTAGE);
  uint8_t* map = (uint8_t*)(smem + 2 * DSTAGE + 16);
  uint32_t* list = (uint32_t*)(map + ((gq + 15) & ~15));

  const int u = remap_unit(blockIdx.x, p.n_units);  // units = B*Hk*NK here
  const int bkv = u / p.NK;                         // b*Hk + kvh
  // the u-th unit in launch order (heaviest key blocks of the head first)
  const int kb = p.korder ? clampi(p.korder[u], 0, p.NK - 1) : u % p.NK;
  const int kvh = bkv % p.Hk;
  const int b = bkv / p.Hk;
  const int64_t kvplane = (int64_t)bkv * p.Sk * HD;
  const int nv = block_valid<BLK>(p.vbs, kb);
  const int key = wave * 16 + r16;  // this lane's key within the block (output)

  const int8_t* mrow = p.k2q + ((int64_t)bkv * p.NK + kb) * gq;  // this block's map row
  for (int i = tid; i < gq; i += NT) map[i] = (uint8_t)mrow[i];
  __syncthreads();
  if (wave == 0) {
    const int n = compact_list(map, gq, list, lane);
    // entry -> first query row (in [B*H*S]) of the listed unit, so the step
    // walk needs no division
    for (int i = lane; i < n; i += 64) {
      const int e = (int)(list[i] >> 8);
      const int hl = e / p.NQ, qb = e - hl * p.NQ;
      const int64_t bh = (int64_t)b * p.H + (int64_t)kvh * p.group + hl;
      list[i] = (uint32_t)(bh * p.S + (int64_t)qb * BLK);
    }
    if (lane == 0) *s_n = n;
  }
  __syncthreads();
  const int nunits = nv > 0 ? *s_n : 0;
  const int nsteps = nunits * QT_PER_UNIT;

  f32x4 dka[8], dva[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dka[dt] = dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A block with at most BLK/2 valid keys would leave the second half of
  // the waves on keys past the count.  Instead those waves take the first
  // half's keys and the second 32 rows of every 64-row query step (the
  // first half keeps rows 0..31); their partial dK, dV are added to the
  // first half's through LDS at the end.  Fixed split, so deterministic.
  const bool halves = 2 * nv <= BLK;
  const int rep = halves && wave >= NW / 2 ? 1 : 0;       // row half (halves)
  const int ckey = (halves ? wave % (NW / 2) : wave) * 16 + r16;  // key computed
  // A wave whose 16 keys all lie past the count only loads and synchronises
  // (its dK, dV stay zero), which leaves its SIMD to the other workgroup.
  const bool active = ckey - r16 < nv;

  if (nsteps > 0) {
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void*)smem;
    // K^T / V^T B operands: column key, rows d = kk*32 + g*8 ..
    bf16x8 kreg[4], vreg[4];
    {
      const int64_t r = kvplane + ((int64_t)kb * BLK + ckey) * HD;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (ckey < nv) {
          kreg[kk] = *(const bf16x8*)(p.k + r + kk * 32 + g * 8);
          vreg[kk] = *(const bf16x8*)(p.v + r + kk * 32 + g * 8);
        } else {
          kreg[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
          vreg[kk] = kreg[kk];
        }
      }
    }
    const int l4 = lane >> 4, pos = lane & 15;
    uint32_t dko[8 / NW];
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const int j = wave + i * NW;
      dko[i] = (uint32_t)(j * 1024 + l4 * ROWB + ((pos ^ bswz(4 * j + l4)) << 4));
    }
    const uint32_t abase = (uint32_t)(r16 * ROWB + ((g ^ bswz(r16)) << 4));
    const uint32_t trb = tr_base(lane);

    // query step t: unit list[t / QT_PER_UNIT], rows (t % QT_PER_UNIT)*64 ..
    auto step_rows = [&](int t) -> int64_t {  // first row in [B*H*S]
      const uint32_t r0 =
          (uint32_t)__builtin_amdgcn_readfirstlane((int)list[t / QT_PER_UNIT]);
      return (int64_t)r0 + (t % QT_PER_UNIT) * QSTEP;
    };
    // Q rows r0..r0+63 -> two tiles, dO likewise, LSE and delta (64 floats
    // each, lanes 0..15 of waves 0 and 1)
    auto issue = [&](int64_t r0, int stg) {
      const uint32_t sl = smem_lds + stg * DSTAGE;
      const char* qg = (const char*)(p.q + r0 * HD);
      const char* dg = (const char*)(p.dout + r0 * HD);
      issue_rows<NW>(qg, sl, dko, wave, l4, KT);
      issue_rows<NW>(qg + TILE_BYTES, sl + TILE_BYTES, dko, wave, l4, KT);
      issue_rows<NW>(dg, sl + 2 * TILE_BYTES, dko, wave, l4, KT);
      issue_rows<NW>(dg + TILE_BYTES, sl + 3 * TILE_BYTES, dko, wave, l4, KT);
      if (wave < 2 && lane < 16) {
        const float* src = wave == 0 ? p.lse : p.delta;
        dma16u((const char*)(src + r0), (uint32_t)lane * 16u,
               sl + (wave == 0 ? LSE_OFF : DLT_OFF));
      }
    };

    // NHF: 32-row halves of each step this wave computes (2, or 1 with
    // `halves`: half hf0 = rep)
    auto run = [&](auto nhf_c) {
      constexpr int NHF = decltype(nhf_c)::value;
      const int hf0 = NHF == 2 ? 0 : rep;
      issue(step_rows(0), 0);
      int t = 0;
      auto step = [&](auto stg_c) -> bool {
        constexpr int STG = decltype(stg_c)::value;
        wait_vm_all();
        __syncthreads();
        const bool has_next = t + 1 < nsteps;
        if (has_next) issue(step_rows(t + 1), STG ^ 1);
        if (!active) {
          if (!has_next) return true;
          ++t;
          return false;
        }
        const char* stage = smem + STG * DSTAGE;
        const char* qtile = stage + hf0 * TILE_BYTES;          // Q rows of half hf0
        const char* dtile = stage + (2 + hf0) * TILE_BYTES;    // dO rows of half hf0
        const char* ltab = stage + LSE_OFF + hf0 * 128;
        const char* dtab = stage + DLT_OFF + hf0 * 128;
        // S and dP for the 16-row query sub-tiles qs (rows qs*16 .. of the
        // wave's halves)
        f32x4 s[2 * NHF], dp[2 * NHF];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int qs = 0; qs < 2 * NHF; ++qs) {
            const uint32_t a =
                (abase ^ (kk << 6)) + (qs & 1) * 16 * ROWB + (qs >> 1) * TILE_BYTES;
            const bf16x8 qop = *(const bf16x8*)(qtile + a);
            const bf16x8 dop = *(const bf16x8*)(dtile + a);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            s[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop, kreg[kk],
                                                            kk == 0 ? z : s[qs], 0, 0, 0);
            dp[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dop, vreg[kk],
                                                             kk == 0 ? z : dp[qs], 0, 0, 0);
          }
        // P and dS as B operands, one pair per 32-row half
        bf16x8 pop[NHF], dsop[NHF];
#pragma unroll
        for (int hf = 0; hf < NHF; ++hf) {
          const f32x4 l0 = *(const f32x4*)(ltab + (hf * 32 + g * 4) * 4);
          const f32x4 l1 = *(const f32x4*)(ltab + (hf * 32 + 16 + g * 4) * 4);
          const f32x4 d0 = *(const f32x4*)(dtab + (hf * 32 + g * 4) * 4);
          const f32x4 d1 = *(const f32x4*)(dtab + (hf * 32 + 16 + g * 4) * 4);
          float pv[8], dsv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int qs = hf * 2 + (e >> 2), j = e & 3;
            const float l = (e >> 2) ? l1[j] : l0[j];
            const float d = (e >> 2) ? d1[j] : d0[j];
            const float pr = ckey < nv ? __builtin_amdgcn_exp2f(
                                             __builtin_fmaf(s[qs][j], p.c, -l))
                                       : 0.f;
            pv[e] = pr;
            dsv[e] = pr * (dp[qs][j] - d);
          }
          pop[hf] = pack8(pv);
          dsop[hf] = pack8(dsv);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint32_t a = trb ^ (uint32_t)(dt << 5);
#pragma unroll
          for (int hf = 0; hf < NHF; ++hf) {
            dva[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                tr_read(dtile + hf * TILE_BYTES, a), pop[hf], dva[dt], 0, 0, 0);
            dka[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                tr_read(qtile + hf * TILE_BYTES, a), dsop[hf], dka[dt], 0, 0, 0);
          }
        }
        if (!has_next) return true;
        ++t;
        return false;
      };
      while (true) {
        if (step(IntC<0>{})) break;
        if (step(IntC<1>{})) break;
      }
    };
    if (halves) {
      run(IntC<1>{});
      // second-half waves hand their partial sums to the first half
      __syncthreads();  // every wave is done with the stages
      f32x4* red = (f32x4*)smem;  // [key group][16][64 lanes]
      const int kg = wave % (NW / 2);
      if (rep == 1) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          red[(kg * 16 + dt) * 64 + lane] = dka[dt];
          red[(kg * 16 + 8 + dt) * 64 + lane] = dva[dt];
          dka[dt] = dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};  // own keys: past the count
        }
      }
      __syncthreads();
      if (rep == 0) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          dka[dt] += red[(kg * 16 + dt) * 64 + lane];
          dva[dt] += red[(kg * 16 + 8 + dt) * 64 + lane];
        }
      }
    } else {
      run(IntC<2>{});
    }
  }

  // dK^T / dV^T: lane holds d = dt*16 + g*4 + j of its key
  const int64_t r = kvplane + ((int64_t)kb * BLK + key) * HD;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const f32x4 kd = dka[dt] * p.sm_scale;
    *(u32x2*)(p.dk + r + dt * 16 + g * 4) =
        u32x2{pack_bf16x2(kd[0], kd[1]), pack_bf16x2(kd[2], kd[3])};
    *(u32x2*)(p.dv + r + dt * 16 + g * 4) =
        u32x2{pack_bf16x2(dva[dt][0], dva[dt][1]), pack_bf16x2(dva[dt][2], dva[dt][3])};
  }
}

// ---------------------------------------------------------------------------
// host side

bool aligned16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

size_t map_bytes(int64_t B, int64_t H, int64_t S, int64_t Sk, int64_t block) {
  return (size_t)(B * H * (S / block) * (Sk / block));
}

size_t delta_bytes(int64_t B, int64_t H, int64_t S) {
  return (size_t)(B * H * S) * sizeof(float);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t map_offset(int64_t B, int64_t H, int64_t S) { return align256(delta_bytes(B, H, S)); }

size_t order_offset(int64_t B, int64_t H, int64_t S, int64_t Sk, int64_t block) {
  return align256(map_offset(B, H, S) + map_bytes(B, H, S, Sk, block));
}

size_t korder_offset(int64_t B, int64_t H, int64_t S, int64_t Sk, int64_t block) {
  return align256(order_offset(B, H, S, Sk, block) +
                  (size_t)(B * H * (S / block)) * sizeof(int32_t));
}

size_t workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t Sk, int64_t block) {
  // delta, the byte map, the dq and the dk/dv launch orders (the latter
  // sized for H >= Hk K/V heads), each 256-byte aligned
  return korder_offset(B, H, S, Sk, block) +
         (size_t)(B * H * (Sk / block)) * sizeof(int32_t);
}

// Static checks of the tensors and sizes (everything but the workspace).
bsa_status check_bwd_args(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, const void* dq,
                          const void* dk, const void* dv, int32_t B, int32_t H,
                          int32_t Hk, int32_t S, int32_t Sk, int32_t D, int32_t block) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return BSA_ERR_NULL;
  if (B <= 0 || H <= 0 || Hk <= 0 || S <= 0 || Sk <= 0 || D <= 0 || block <= 0)
    return BSA_ERR_SHAPE;
  if (S % block != 0 || Sk % block != 0 || H % Hk != 0) return BSA_ERR_SHAPE;
  if (D != HD || (block != 64 && block != 128)) return BSA_ERR_UNSUPPORTED;
  if (Sk / block > BSA_MAX_KEY_BLOCKS) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)(H / Hk) * (S / block) > BSA_MAX_KEY_BLOCKS) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * H * S > INT32_MAX || (int64_t)B * Hk * Sk > INT32_MAX)
    return BSA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(dout) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return BSA_ERR_ALIGN;
  return BSA_OK;
}

bsa_status check_bwd(const void* q, const void* k, const void* v, const void* out,
                     const void* dout, const float* lse, const void* dq,
                     const void* dk, const void* dv, const void* ws,
                     int32_t B, int32_t H, int32_t Hk, int32_t S, int32_t Sk,
                     int32_t D, int32_t block) {
  if (!ws) return BSA_ERR_NULL;
  const bsa_status st = check_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, B, H, Hk, S,
                                       Sk, D, block);
  if (st != BSA_OK) return st;
  if (((uintptr_t)ws & 255u) != 0) return BSA_ERR_ALIGN;
  return BSA_OK;
}

template <int BLK, bool BITMAP>
bsa_status run_bwd(BwdParams p, const void* out, float* delta, int8_t* map,
                   size_t nmap, int32_t* order, int32_t* korder, int32_t B,
                   hipStream_t st) {
  // LUT form: dq units launched heaviest first within each (b, h), as the
  // forward pass does (same order pass; no effect on the result)
  p.order = nullptr;
  if (!BITMAP && p.NQ <= BSA_MAX_ORDER_QBLOCKS && p.n_units > ORDER_MIN_UNITS) {
    const bsa_status os = bsa_unit_order_lut(p.idx, p.num, p.max_kv, p.meta_sb, p.meta_sh,
                                             p.vbs, order, B, p.H, p.S, p.Sk,
                                             p.S / p.NQ, (void*)st);
    if (os != BSA_OK) return os;
    p.order = order;
  }
  const int64_t rows = (int64_t)p.n_units * BLK;  // B*H*S
  hipLaunchKernelGGL(delta_kernel, dim3((uint32_t)((rows + 15) / 16)), dim3(256), 0, st,
                     (const uint16_t*)out, p.dout, delta, rows);
  if ((nmap & 15) == 0 && ((uintptr_t)map & 15) == 0)
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, st, (u32x4*)map,
                       (int64_t)(nmap / 16));
  else
    hipLaunchKernelGGL(fill_zero_bytes_kernel, dim3(1024), dim3(256), 0, st, map,
                       (int64_t)nmap);
  p.delta = delta;
  p.k2q = map;
  hipLaunchKernelGGL(k2q_kernel<BITMAP>, dim3((uint32_t)((p.n_units + 3) / 4)), dim3(256),
                     0, st, p);
  {
    auto kern = dq_kernel<BLK, BITMAP>;
    const size_t lds = 2 * BSTAGE + 16 + (size_t)((p.NK + 15) & ~15) + (size_t)p.NK * 4;
    if (lds > 65536 && hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
    hipLaunchKernelGGL(kern, dim3(p.n_units), dim3(BLK * 2), lds, st, p);
  }
  {
    auto kern = dkdv_kernel<BLK>;
    const int gq = p.group * p.NQ;
    const size_t lds = 2 * DSTAGE + 16 + (size_t)((gq + 15) & ~15) + (size_t)gq * 4;
    if (lds > 65536 && hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds) != hipSuccess)
      return BSA_ERR_HIP;
    BwdParams pk = p;
    pk.n_units = (int32_t)((int64_t)p.n_units / p.H * p.Hk / p.NQ * p.NK);
    // key blocks of each (b, K/V head) launched heaviest first
    pk.korder = nullptr;
    if (p.NK <= BSA_MAX_ORDER_QBLOCKS && pk.n_units > ORDER_MIN_UNITS) {
      hipLaunchKernelGGL(kunit_work_kernel, dim3((uint32_t)((pk.n_units + 3) / 4)),
                         dim3(256), 0, st, pk, korder, pk.n_units);
      const bsa_status rs = bsa_rank_runs(korder, pk.n_units / p.NK, p.NK, st);
      if (rs != BSA_OK) return rs;
      pk.korder = korder;
    }
    hipLaunchKernelGGL(kern, dim3(pk.n_units), dim3(BLK * 4), lds, st, pk);
  }
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

BwdParams make_bwd_params(const void* q, const void* k, const void* v,
                          const void* dout, const float* lse,
                          const int32_t* vbs, float sm_scale, void* dq, void* dk,
                          void* dv, int32_t B, int32_t H, int32_t Hk, int32_t S,
                          int32_t Sk, int32_t block) {
  BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.vbs = vbs;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.sm_scale = sm_scale;
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

template <bool BITMAP>
bsa_status dispatch_bwd(const BwdParams& p, int block, const void* out, void* ws,
                        size_t ws_bytes, int32_t B, int32_t H, int32_t S, int32_t Sk,
                        hipStream_t st) {
  const size_t need = workspace_bytes(B, H, S, Sk, block);
  if (ws_bytes < need) return BSA_ERR_SHAPE;
  float* delta = (float*)ws;
  int8_t* map = (int8_t*)ws + map_offset(B, H, S);
  const size_t nmap = map_bytes(B, H, S, Sk, block);
  int32_t* order = (int32_t*)((char*)ws + order_offset(B, H, S, Sk, block));
  int32_t* korder = (int32_t*)((char*)ws + korder_offset(B, H, S, Sk, block));
  if (block == 64)
    return run_bwd<64, BITMAP>(p, out, delta, map, nmap, order, korder, B, st);
  return run_bwd<128, BITMAP>(p, out, delta, map, nmap, order, korder, B, st);
}

}  // namespace

extern "C" size_t bsa_bwd_workspace_size(int32_t B, int32_t H, int32_t S, int32_t Sk,
                                         int32_t block) {
  if (B <= 0 || H <= 0 || S <= 0 || Sk <= 0 || block <= 0) return 0;
  return workspace_bytes(B, H, S, Sk, block);
}

extern "C" bsa_status bsa_bwd_lut(const void* q, const void* k, const void* v,
                                  const void* out, const void* dout, const float* lse,
                                  const int32_t* q2k_idx, const int32_t* q2k_num,
                                  int32_t max_kv, int64_t meta_stride_b,
                                  int64_t meta_stride_h,
                                  const int32_t* variable_block_sizes, float sm_scale,
                                  void* dq, void* dk, void* dv, void* workspace,
                                  size_t workspace_bytes_, int32_t B, int32_t H,
                                  int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                                  int32_t block, void* stream) {
  bsa_status st = check_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Hk, S,
                            Sk, D, block);
  if (st != BSA_OK) return st;
  if (!__builtin_isfinite(sm_scale)) return BSA_ERR_VALUE;
  if (!q2k_idx || !q2k_num) return BSA_ERR_NULL;
  if (max_kv < 1 || meta_stride_b < 0 || meta_stride_h < 0) return BSA_ERR_SHAPE;
  BwdParams p = make_bwd_params(q, k, v, dout, lse, variable_block_sizes, sm_scale, dq,
                                dk, dv, B, H, Hk, S, Sk, block);
  p.idx = q2k_idx;
  p.num = q2k_num;
  p.max_kv = max_kv;
  p.meta_sb = meta_stride_b;
  p.meta_sh = meta_stride_h;
  return dispatch_bwd<false>(p, block, out, workspace, workspace_bytes_, B, H, S, Sk,
                             (hipStream_t)stream);
}

extern "C" bsa_status bsa_bwd_bitmap(const void* q, const void* k, const void* v,
                                     const void* out, const void* dout,
                                     const float* lse, const int8_t* mask,
                                     int64_t mask_stride_b, int64_t mask_stride_h,
                                     const int32_t* variable_block_sizes, float sm_scale,
                                     void* dq, void* dk, void* dv, void* workspace,
                                     size_t workspace_bytes_, int32_t B, int32_t H,
                                     int32_t Hk, int32_t S, int32_t Sk, int32_t D,
                                     int32_t block, void* stream) {
  bsa_status st = check_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Hk, S,
                            Sk, D, block);
  if (st != BSA_OK) return st;
  if (!__builtin_isfinite(sm_scale)) return BSA_ERR_VALUE;
  if (!mask) return BSA_ERR_NULL;
  if (mask_stride_b < 0 || mask_stride_h < 0) return BSA_ERR_SHAPE;
  BwdParams p = make_bwd_params(q, k, v, dout, lse, variable_block_sizes, sm_scale, dq,
                                dk, dv, B, H, Hk, S, Sk, block);
  p.mask = mask;
  p.meta_sb = mask_stride_b;
  p.meta_sh = mask_stride_h;
  return dispatch_bwd<true>(p, block, out, workspace, workspace_bytes_, B, H, S, Sk,
                            (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// Allocation-free backward entry point: the workspace is the library's own
// device array, one copy per GPU (allocated when the library's code object
// is loaded on that GPU, held until the process ends).  Host code uses the
// array only through its device address, taken once per device.

static __device__ __align__(256) char scratch[BSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// Device address of `scratch` on the current device.
bsa_status scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return BSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BSA_OK;
}

}  // namespace

extern "C" bsa_status bsa_bwd_lut_noalloc(const void* q, const void* k, const void* v,
                                          const void* out, const void* dout,
                                          const float* lse, const int32_t* q2k_idx,
                                          const int32_t* q2k_num, int32_t max_kv,
                                          int64_t meta_stride_b, int64_t meta_stride_h,
                                          const int32_t* variable_block_sizes,
                                          float sm_scale, void* dq, void* dk, void* dv,
                                          int32_t B, int32_t H, int32_t Hk, int32_t S,
                                          int32_t Sk, int32_t D, int32_t block,
                                          void* stream) {
  bsa_status st = check_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, B, H, Hk, S, Sk, D,
                                 block);
  if (st != BSA_OK) return st;
  if (!__builtin_isfinite(sm_scale)) return BSA_ERR_VALUE;
  if (!q2k_idx || !q2k_num) return BSA_ERR_NULL;
  if (max_kv < 1 || meta_stride_b < 0 || meta_stride_h < 0) return BSA_ERR_SHAPE;
  if (workspace_bytes(B, H, S, Sk, block) > (size_t)BSA_NOALLOC_SCRATCH_BYTES)
    return BSA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BSA_OK) return st;
  return bsa_bwd_lut(q, k, v, out, dout, lse, q2k_idx, q2k_num, max_kv, meta_stride_b,
                     meta_stride_h, variable_block_sizes, sm_scale, dq, dk, dv, ws,
                     (size_t)BSA_NOALLOC_SCRATCH_BYTES, B, H, Hk, S, Sk, D, block, stream);
}
