// bsa_device.h -- device helpers shared by the gfx950 attention kernels
// (forward, backward): tile geometry, bf16 packing, cross-lane reductions,
// the selected-block list reader and the direct global->LDS tile loads.
#ifndef BSA_DEVICE_H
#define BSA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"

namespace {

constexpr int HD = 128;                 // head dimension
constexpr int KT = 32;                  // rows per pipeline tile
constexpr int ROWB = HD * 2;            // bytes of one bf16 row in LDS
constexpr int TILE_BYTES = KT * ROWB;   // one 32-row tile (8 KB)
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Compile-time integer as a type (selects unrolled loop variants).
template <int V>
struct IntC {
  static constexpr int value = V;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Valid keys of key block kb.
template <int BLK>
__device__ __forceinline__ int block_valid(const int32_t* vbs, int kb) {
  return vbs ? clampi(vbs[kb], 0, BLK) : BLK;
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  Give XCD x the
// contiguous unit range [x*n/8, (x+1)*n/8) so the units of one head (and of
// the query heads that share its K/V head), which read the same K/V blocks,
// meet in the same L2.
__device__ __forceinline__ int remap_unit(int bid, int n) {
  if (n % 8 != 0) return bid;
  return (bid % 8) * (n / 8) + bid / 8;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 r = __builtin_convertvector(f, bf16x2);  // v_cvt_pk_bf16_f32, RNE
  return __builtin_bit_cast(uint32_t, r);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the lanes that hold
// one query row), with the gfx950 cross-row lane swaps (no LDS traffic).
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_min(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  x = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return fmaxf(fmaxf(a, b), c);
}

// Position of one pipeline tile: entry e of the selected-block list, first
// key t0 within the block, valid keys nv of the block.
struct Tile {
  int e, kb, t0, nv;
};

// Reader of the selected-block list ((kb << 8) | nv per entry, nv = valid
// keys).  Entries are fetched from LDS 64 at a time into one VGPR (lane i
// holds entry base + i) and picked out with v_readlane, so moving to the
// next block costs no LDS round trip on the critical path.  The following
// 64 entries are fetched one chunk ahead (into `ahead`): a chunk is read
// long after its load was issued, so the walk never waits on the LDS
// counter, which would also wait for every LDS read issued before it (the
// K operand reads of the tile in hand).
struct ListCursor {
  const uint32_t* list;
  int nsel;
  int base;
  uint32_t chunk;
  uint32_t ahead;

  __device__ __forceinline__ void reset(int lane) {
    base = 0;
    chunk = lane < nsel ? list[lane] : 0u;
    ahead = 64 + lane < nsel ? list[64 + lane] : 0u;
  }

  // Entries are visited in increasing order, one at a time.
  __device__ __forceinline__ Tile at(int e, int lane) {
    Tile t;
    t.e = e;
    t.t0 = 0;
    t.kb = 0;
    t.nv = 0;
    if (e < nsel) {
      if (e >= base + 64) {
        base += 64;
        chunk = ahead;
        ahead = base + 64 + lane < nsel ? list[base + 64 + lane] : 0u;
      }
      const uint32_t x = (uint32_t)__builtin_amdgcn_readlane((int)chunk, e - base);
      t.kb = (int)(x >> 8);
      t.nv = (int)(x & 255u);
    }
    return t;
  }

  __device__ __forceinline__ Tile next(const Tile& cur, int lane) {
    if (cur.t0 + KT < cur.nv) {
      Tile t = cur;
      t.t0 += KT;
      return t;
    }
    return at(cur.e + 1, lane);
  }
};

// Position in the stream of a unit's valid keys (each selected block's
// valid keys, blocks in list order): entry e of the list, key o of that
// entry's block.
struct Walk {
  int e, o;
};

// Cuts the 32-row tile that starts at stream position w (w.e < nsel),
// moves w past it and returns its row count (1..32).  When all 32 rows lie
// in one block, row rr holds key key0 + rr and full(key0) issues the loads.
// Otherwise rows [0, rows) hold the next `rows` keys of the stream, which
// may come from several blocks: a run of rows that starts at tile row r0 in
// block kb holds keys kb*BLK + rr - r0, so a lane whose row rr (rows
// 4j .. 4j+3 of slice i, j = wave + i*NW) falls in that run sits
// ex[i] = (kb*BLK - r0 - key0) rows past key0 + rr (>= 0: keys ascend along
// the stream); split(key0, rows, ex) issues the loads.
// Lane offsets are 32-bit byte offsets from key0's row; they stay below
// one head's K/V plane, at most BSA_MAX_KEY_BLOCKS blocks of 128 keys.
static_assert((int64_t)BSA_MAX_KEY_BLOCKS * 128 * ROWB < ((int64_t)1 << 32),
              "stream-tile lane offsets must fit 32 bits");

template <int BLK, int NW, class Full, class Split>
__device__ __forceinline__ int next_stream_tile(ListCursor& cursor, Walk& w, int nsel,
                                                int wave, int l4, int lane, Full&& full,
                                                Split&& split) {
  const Tile t = cursor.at(w.e, lane);
  const int avail = t.nv - w.o;
  const int64_t key0 = (int64_t)t.kb * BLK + w.o;
  if (avail >= KT) {
    w.o += KT;
    if (w.o >= t.nv) {
      ++w.e;
      w.o = 0;
    }
    full(key0);
    return KT;
  }
  int row = avail;
  ++w.e;
  w.o = 0;
  uint32_t ex[8 / NW];
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) ex[i] = 0u;
  while (row < KT && w.e < nsel) {
    const Tile u = cursor.at(w.e, lane);
    const int take = min(u.nv, KT - row);
    const uint32_t d = (uint32_t)((int64_t)u.kb * BLK - row - key0) << 8;
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i)
      ex[i] = l4 >= row - 4 * (wave + i * NW) ? d : ex[i];
    row += take;
    if (take == u.nv) {
      ++w.e;
    } else {
      w.o = take;
    }
  }
  split(key0, row, ex);
  return row;
}

// One direct global->LDS load of 16 B per lane (global_load_lds_dwordx4,
// SGPR base + 32-bit VGPR offset): lane l's 16 bytes land at LDS address
// lds_base + 16*l.  Issued as inline assembly so that the compiler does not
// track it; the loop waits for these loads explicitly (vmcnt) before the
// barrier that publishes a tile, and the reads of the other stage proceed
// while they are in flight.
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff,
                                      uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_base), "v"(voff), "s"(gbase)
      : "memory", "m0");
}

// dma16 for callers whose bases the compiler cannot prove wave-uniform
// (they are): readfirstlane pins them to SGPRs.
__device__ __forceinline__ void dma16u(const char* gbase, uint32_t voff,
                                       uint32_t lds_base) {
  const uint64_t gb = (uint64_t)(uintptr_t)gbase;
  // readfirstlane returns int: go through uint32_t so nothing sign-extends
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gb >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gb);
  const uint64_t gs = ((uint64_t)hi << 32) | (uint64_t)lo;
  dma16((const char*)(uintptr_t)gs, voff,
        (uint32_t)__builtin_amdgcn_readfirstlane(lds_base));
}

// Waits until this wave's outstanding global loads (including the ones
// writing LDS directly) have completed.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
}

// Direct loads of one 32-row bf16 tile (8 KB) shared by the NW waves of a
// workgroup.  The tile's 8 slices of 4 rows (1 KB) are dealt round-robin:
// slice j = wave + i*NW lands at LDS dst + j*1024; lane l fills LDS
// position l & 15 of row 4j + l/16 from global offset off[i] (row offset
// and swizzle folded in, fixed per lane).  With nv < 32 valid rows, lanes of
// rows at or past nv re-read the chunk at the same position of the tile's
// row 0 (a valid row), so the load count is fixed and no row past nv is
// ever read.
template <int NW>
__device__ __forceinline__ void issue_rows(const char* g, uint32_t dst,
                                           const uint32_t (&off)[8 / NW],
                                           int wave, int l4, int nv) {
  if (nv >= KT) {
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i)
      dma16u(g, off[i], dst + (uint32_t)(wave + i * NW) * 1024u);
  } else {
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const int j = wave + i * NW;
      dma16u(g, 4 * j + l4 < nv ? off[i] : (off[i] & 0xFFu), dst + (uint32_t)j * 1024u);
    }
  }
}

// issue_rows for a tile of the key stream that spans blocks or is partial
// (see next_stream_tile): g is key0's row; lanes of rows past the count
// re-read row 0's chunk.
template <int NW>
__device__ __forceinline__ void issue_split_rows(const char* g, uint32_t dst,
                                                 const uint32_t (&off)[8 / NW],
                                                 const uint32_t (&ex)[8 / NW], int rows,
                                                 int wave, int l4) {
#pragma unroll
  for (int i = 0; i < 8 / NW; ++i) {
    const int j = wave + i * NW;
    dma16u(g, 4 * j + l4 < rows ? off[i] + ex[i] : (off[i] & 0xFFu), dst + (uint32_t)j * 1024u);
  }
}

}  // namespace

#endif  // BSA_DEVICE_H
