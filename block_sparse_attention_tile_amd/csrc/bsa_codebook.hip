// bsa_codebook.hip -- codebook K/V dequantisation for MI355X (gfx950).
//
// rocke "sage_attention.py" (module docstring and its codebook-dequant
// primitives) stores K/V as small integer codes that index an f32 codebook:
// i8 codes at code + 128 in a 256-entry table, i4 codes packed two per byte
// (element 2i in the low nibble, two's complement) at code + 8 in a
// 16-entry table; the per-block scale multiplies the looked-up value.
//
// This pass turns codes into bf16 codebook values (RNE) once per call; the
// forward pass then reads them as BSA_KV_BF16_SCALED, applying the
// per-block scale exactly as it does for fp8.  For block-sparse attention
// every K/V block is gathered by many query units, so one lookup per
// element here replaces one per element and per gathering unit inside the
// attention kernel.  HBM-bound: 1 B (i8) or 0.5 B (i4) read and 2 B
// written per element.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bsa.h"
#include "bsa_device.h"

namespace {

// One workgroup turns 8192 consecutive codes into bf16 values: each thread
// takes four groups of 8 codes, 256 groups apart, so that every load and
// every 16-byte store of a wave covers one contiguous span, and all four
// loads are in flight before the first lookup.  The bf16-rounded codebook
// sits in LDS: for i8 one 16-bit entry per level, where the level of a code
// byte is (code + 128) = byte ^ 0x80; for i4 one 32-bit entry per code byte
// holding both of its values, the level of a nibble being (code + 8) =
// nibble ^ 8.
constexpr int DQ_R = 4;                 // groups of 8 codes per thread
constexpr int DQ_GROUPS = 256 * DQ_R;   // groups per workgroup

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const f32x2 f = {x, 0.f};
  const bf16x2 r = __builtin_convertvector(f, bf16x2);  // RNE
  return (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xFFFFu);
}

template <int KIND>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ codebook,
                                                      uint16_t* __restrict__ out,
                                                      int64_t groups) {
  constexpr bool I8 = KIND == BSA_CODEBOOK_I8;
  using Word = std::conditional_t<I8, u32x2, uint32_t>;  // 8 codes
  __shared__ std::conditional_t<I8, uint16_t, uint32_t> tab[256];
  const int tid = threadIdx.x;
  const int64_t g0 = (int64_t)blockIdx.x * DQ_GROUPS + tid;
  Word w[DQ_R];
#pragma unroll
  for (int r = 0; r < DQ_R; ++r) {
    const int64_t gi = g0 + r * 256;
    if (gi < groups) w[r] = ((const Word*)codes)[gi];
  }
  if constexpr (I8) {
    tab[tid] = bf16_rne(codebook[tid]);
  } else {
    tab[tid] = (uint32_t)bf16_rne(codebook[(tid & 15) ^ 8]) |
               ((uint32_t)bf16_rne(codebook[(tid >> 4) ^ 8]) << 16);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < DQ_R; ++r) {
    const int64_t gi = g0 + r * 256;
    if (gi >= groups) break;
    u32x4 o;
    if constexpr (I8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[r][i >> 1] >> (16 * (i & 1));
        o[i] = (uint32_t)tab[(x & 0xFFu) ^ 0x80u] |
               ((uint32_t)tab[((x >> 8) & 0xFFu) ^ 0x80u] << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = tab[(w[r] >> (8 * i)) & 0xFFu];
    }
    ((u32x4*)out)[gi] = o;
  }
}

}  // namespace

extern "C" bsa_status bsa_codebook_dequant(const void* codes, int32_t kind,
                                           const float* codebook, void* out,
                                           int64_t n_values, void* stream) {
  if (kind != BSA_CODEBOOK_I8 && kind != BSA_CODEBOOK_I4) return BSA_ERR_UNSUPPORTED;
  if (n_values < 0 || n_values % 16 != 0) return BSA_ERR_SHAPE;
  if (n_values == 0) return BSA_OK;
  if (!codes || !codebook || !out) return BSA_ERR_NULL;
  const uintptr_t calign = kind == BSA_CODEBOOK_I8 ? 15u : 7u;
  if (((uintptr_t)codes & calign) != 0 || ((uintptr_t)out & 15u) != 0)
    return BSA_ERR_ALIGN;
  const int64_t groups = n_values / 8;
  const int64_t blocks = (groups + DQ_GROUPS - 1) / DQ_GROUPS;
  if (blocks > INT32_MAX) return BSA_ERR_UNSUPPORTED;
  const dim3 grid((uint32_t)blocks);
  if (kind == BSA_CODEBOOK_I8)
    hipLaunchKernelGGL(dequant_kernel<BSA_CODEBOOK_I8>, grid, dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)codes, codebook,
                       (uint16_t*)out, groups);
  else
    hipLaunchKernelGGL(dequant_kernel<BSA_CODEBOOK_I4>, grid, dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)codes, codebook,
                       (uint16_t*)out, groups);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}
