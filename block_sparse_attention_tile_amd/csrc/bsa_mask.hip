// bsa_mask.hip -- block-map -> look-up-table compaction for MI355X (gfx950).
//
// Turns a per-row key-block bitmap (i8, nonzero = attend; the Jenga form of
// rocke "sparse_attention.py") into the VSA form consumed by bsa_fwd_lut:
// q2k_idx holds the row's selected key blocks in ascending order followed by
// -1 padding, q2k_num the count.  This is the step FastVideo
// "block_sparse_attn_sm100a.py" performs with `map_to_index` before its
// from-mask launch (`block_sparse_attn_sm100a_from_mask`); the padding is
// never read by the forward pass (`is_supported` docstring).
//
// One wave per row.  Each pass over the row covers 1024 key blocks: every
// lane loads 16 consecutive mask bytes at once (a row of up to 1024 blocks
// is one load per lane, so a wave waits for memory once), the wave forms
// the exclusive prefix of the per-lane counts (0..16) with five ballots
// (count = sum of 2^b over its bits b), and each lane writes its selected
// indices at their final positions.  The padding is then written with one
// store per lane per 64 entries.  Integer work only: the result is exact.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"

namespace {

constexpr int WAVES = 4;    // rows per workgroup
constexpr int PER_LANE = 16;  // mask bytes per lane and pass
constexpr int CHUNK = 64 * PER_LANE;  // key blocks per wave pass

__device__ __forceinline__ int prefix_lt(uint64_t ballot) {
  // number of set bits of `ballot` in lanes below this one
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0));
}

// bit i of the result: byte i of w is nonzero (i < 4)
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) b |= ((w >> (8 * i)) & 0xFFu) ? (1u << i) : 0u;
  return b;
}

__global__ __launch_bounds__(WAVES * 64) void mask_to_lut_kernel(
    const int8_t* __restrict__ mask, int64_t rows, int32_t nk,
    int32_t* __restrict__ idx, int32_t* __restrict__ num) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves together
  const int8_t* m = mask + row * nk;
  int32_t* out = idx + row * nk;
  const bool aligned16 = ((uintptr_t)m & 15u) == 0;
  const bool aligned4 = ((uintptr_t)m & 3u) == 0;

  int n = 0;  // entries written so far (wave-uniform)
  for (int base = 0; base < nk; base += CHUNK) {
    const int k0 = base + PER_LANE * lane;
    uint32_t bits = 0;  // bit i: key block k0 + i selected
    if (aligned16 && k0 + PER_LANE <= nk) {
      const uint4 w = *(const uint4*)(m + k0);
      bits = nonzero_bytes(w.x) | (nonzero_bytes(w.y) << 4) | (nonzero_bytes(w.z) << 8) |
             (nonzero_bytes(w.w) << 12);
    } else if (aligned4 && k0 + PER_LANE <= nk) {
      const uint32_t* m4 = (const uint32_t*)(m + k0);
#pragma unroll
      for (int i = 0; i < PER_LANE / 4; ++i) bits |= nonzero_bytes(m4[i]) << (4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (k0 + i < nk && m[k0 + i] != 0) bits |= 1u << i;
    }
    const int cnt = __builtin_popcount(bits);
    int pos = n, total = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const uint64_t bal = __ballot((cnt >> b) & 1);
      pos += prefix_lt(bal) << b;
      total += __popcll(bal) << b;
    }
    while (bits) {
      out[pos++] = k0 + __builtin_ctz(bits);
      bits &= bits - 1u;
    }
    n += total;
  }
  // padding: single entries up to a 16-byte boundary, then 16-byte stores
  int j0 = n;
  while (j0 < nk && ((uintptr_t)(out + j0) & 15u) != 0) ++j0;  // at most 3 steps
  if (n + lane < j0) out[n + lane] = -1;
  const int nq = (nk - j0) >> 2;  // whole 4-entry groups
  int4* o4 = (int4*)(out + j0);
  for (int q = lane; q < nq; q += 64) o4[q] = int4{-1, -1, -1, -1};
  for (int j = j0 + 4 * nq + lane; j < nk; j += 64) out[j] = -1;
  if (lane == 0) num[row] = n;
}

}  // namespace

extern "C" bsa_status bsa_mask_to_lut(const int8_t* mask, int64_t rows,
                                      int32_t nk, int32_t* q2k_idx,
                                      int32_t* q2k_num, void* stream) {
  if (rows < 0 || nk <= 0) return BSA_ERR_SHAPE;
  if (nk > BSA_MAX_KEY_BLOCKS) return BSA_ERR_UNSUPPORTED;
  if (rows == 0) return BSA_OK;
  if (!mask || !q2k_idx || !q2k_num) return BSA_ERR_NULL;
  const int64_t blocks = (rows + WAVES - 1) / WAVES;
  if (blocks > INT32_MAX) return BSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mask_to_lut_kernel, dim3((uint32_t)blocks), dim3(WAVES * 64), 0,
                     (hipStream_t)stream, mask, rows, nk, q2k_idx, q2k_num);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}
