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

#include "bsa.h"
#include "bsa_device.h"

namespace {

// One thread turns 16 consecutive codes into 16 bf16 values (32 bytes).
// The table is the codebook rounded to bf16, staged in LDS.  The level of
// an i8 code is (code + 128) = byte ^ 0x80; of an i4 nibble (code + 8) =
// nibble ^ 8.
template <int KIND>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ codebook,
                                                      uint16_t* __restrict__ out,
                                                      int64_t groups) {
  constexpr int NENT = KIND == BSA_CODEBOOK_I8 ? 256 : 16;
  __shared__ uint16_t tab[NENT];
  for (int i = threadIdx.x; i < NENT; i += 256) {
    const f32x2 f = {codebook[i], 0.f};
    const bf16x2 r = __builtin_convertvector(f, bf16x2);  // RNE
    tab[i] = (uint16_t)(__builtin_bit_cast(uint32_t, r) & 0xFFFFu);
  }
  __syncthreads();
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * 256) {
    uint32_t lv[16];  // table levels of the 16 codes
    if constexpr (KIND == BSA_CODEBOOK_I8) {
      const u32x4 w = ((const u32x4*)codes)[gi];
#pragma unroll
      for (int i = 0; i < 16; ++i) lv[i] = ((w[i >> 2] >> (8 * (i & 3))) & 0xFFu) ^ 0x80u;
    } else {
      const u32x2 w = ((const u32x2*)codes)[gi];
#pragma unroll
      for (int i = 0; i < 16; ++i) lv[i] = ((w[i >> 3] >> (4 * (i & 7))) & 0xFu) ^ 0x8u;
    }
    u32x4 o0, o1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o0[i] = (uint32_t)tab[lv[2 * i]] | ((uint32_t)tab[lv[2 * i + 1]] << 16);
      o1[i] = (uint32_t)tab[lv[8 + 2 * i]] | ((uint32_t)tab[lv[8 + 2 * i + 1]] << 16);
    }
    ((u32x4*)out)[2 * gi] = o0;
    ((u32x4*)out)[2 * gi + 1] = o1;
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
  const int64_t groups = n_values / 16;
  const int64_t want = (groups + 255) / 256;
  const uint32_t grid = (uint32_t)(want < 8192 ? want : 8192);
  if (kind == BSA_CODEBOOK_I8)
    hipLaunchKernelGGL(dequant_kernel<BSA_CODEBOOK_I8>, dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)codes, codebook,
                       (uint16_t*)out, groups);
  else
    hipLaunchKernelGGL(dequant_kernel<BSA_CODEBOOK_I4>, dim3(grid), dim3(256), 0,
                       (hipStream_t)stream, (const uint8_t*)codes, codebook,
                       (uint16_t*)out, groups);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}
