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
// One wave per row.  Each pass over the row covers 256 key blocks: every
// lane tests 4 consecutive mask bytes, the wave forms the exclusive prefix
// of the per-lane counts with three ballots (count = b0 + 2 b1 + 4 b2), and
// each lane writes its selected indices at their final positions.  The
// padding is then written with one store per lane per 64 entries.  Integer
// work only: the result is exact.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"

namespace {

constexpr int WAVES = 4;  // rows per workgroup
constexpr int CHUNK = 256;  // key blocks per wave pass (64 lanes x 4)

__device__ __forceinline__ int prefix_lt(uint64_t ballot) {
  // number of set bits of `ballot` in lanes below this one
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)ballot, 0));
}

__global__ __launch_bounds__(WAVES * 64) void mask_to_lut_kernel(
    const int8_t* __restrict__ mask, int64_t rows, int32_t nk,
    int32_t* __restrict__ idx, int32_t* __restrict__ num) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves together
  const int8_t* m = mask + row * nk;
  int32_t* out = idx + row * nk;
  const bool aligned = ((uintptr_t)m & 3u) == 0;

  int n = 0;  // entries written so far (wave-uniform)
  for (int base = 0; base < nk; base += CHUNK) {
    const int k0 = base + 4 * lane;
    uint32_t bits = 0;  // bit i: key block k0 + i selected
    if (aligned && k0 + 4 <= nk) {
      const uint32_t w = *(const uint32_t*)(m + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) bits |= ((w >> (8 * i)) & 0xFFu) ? (1u << i) : 0u;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k0 + i < nk && m[k0 + i] != 0) bits |= 1u << i;
    }
    const int cnt = __builtin_popcount(bits);
    const uint64_t b0 = __ballot(cnt & 1);
    const uint64_t b1 = __ballot(cnt & 2);
    const uint64_t b2 = __ballot(cnt & 4);
    int pos = n + prefix_lt(b0) + 2 * prefix_lt(b1) + 4 * prefix_lt(b2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (bits & (1u << i)) out[pos++] = k0 + i;
    n += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
  }
  for (int j = n + lane; j < nk; j += 64) out[j] = -1;
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
