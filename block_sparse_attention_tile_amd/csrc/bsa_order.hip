// bsa_order.hip -- work order of the forward launch (both forms).
//
// Work units are independent: unit (b, h, qb) computes the same bits
// whichever workgroup slot runs it and whenever it runs.  Their cost is
// not equal, though: it grows with the unit's attended keys (the valid keys
// of its selected key blocks, FastVideo "block_sparse_attn_sm100a.py",
// `is_supported` docstring: counts in [0, max_kv], keys past a block's
// `variable_block_sizes` entry masked).  Launched in q-block order, units
// that happen to be heavy and start late leave a tail in which most slots
// idle.  This pass orders the q-blocks of every (b, h) by decreasing
// attended-key count, so that the forward launch starts its heavy units
// first and runs units of similar length side by side (they then also stay
// at the same point of their ascending key sweeps, which keeps the K/V they
// share in L2).  Two kernels:
//   1. one wave per unit: work = sum over the row's first clamp(num, 0,
//      max_kv) LUT entries inside [0, NK) of the block's valid keys (a cost
//      estimate: a repeated entry is counted twice), or over the blocks its
//      mask row selects (bitmap form, exact); the rank value is
//      min(work / 64, 2^21 - 1) * 1024 + 1023 - mean, mean = the entries'
//      average block index scaled to 0..1023 (truncated): counts in the
//      same 64-key bucket order by where their selection lies;
//   2. one workgroup per (b, h): each q-block's position is the rank of its
//      64-bit key ((2^32 - 1 - work) << 32 | qb) among the NQ keys in LDS.
// The result is deterministic (no atomics) and only affects scheduling.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa.h"
#include "bsa_device.h"

namespace {

struct OrderParams {
  const int32_t* idx;
  const int32_t* num;
  const int8_t* mask;  // [rows, NK] (bitmap form) or null
  int32_t max_kv;
  int64_t meta_sb;
  int64_t meta_sh;
  const int32_t* vbs;  // [NK] or null
  int32_t* order;      // [B*H*NQ]: work after kernel 1, q-blocks after kernel 2
  int32_t H;
  int32_t NQ;
  int32_t NK;
  int32_t block;
  int32_t n_units;
};

// Sums of a wave's per-lane (valid keys, block index, entries) and the
// unit's rank value: valid keys in buckets of 64 (units within a bucket run
// about equally long), then the mean selected block scaled to 0..1023, lower
// first (units that start their sweeps alike run side by side).
__device__ __forceinline__ void store_rank(const OrderParams& p, int u, int lane,
                                           long long w, long long ps, long long cnt) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    w += __shfl_xor(w, o);
    ps += __shfl_xor(ps, o);
    cnt += __shfl_xor(cnt, o);
  }
  const long long bucket = w >> 6 < (1ll << 21) - 1 ? w >> 6 : (1ll << 21) - 1;
  const long long mean = cnt ? ps * 1023 / (cnt * (p.NK > 1 ? p.NK - 1 : 1)) : 0;
  if (lane == 0) p.order[u] = (int32_t)((bucket << 10) | (1023 - mean));
}

__global__ __launch_bounds__(256) void unit_work_kernel(OrderParams p) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= p.n_units) return;
  const int qb = u % p.NQ;
  const int bh = u / p.NQ;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int64_t row = (int64_t)b * p.meta_sb + (int64_t)h * p.meta_sh + qb;
  const int n = clampi(p.num[row], 0, p.max_kv);
  const int32_t* irow = p.idx + row * p.max_kv;
  long long w = 0, ps = 0, cnt = 0;
  for (int j = lane; j < n; j += 64) {
    const int kb = irow[j];
    if (kb >= 0 && kb < p.NK) {
      w += p.vbs ? clampi(p.vbs[kb], 0, p.block) : p.block;
      ps += kb;
      cnt += 1;
    }
  }
  store_rank(p, u, lane, w, ps, cnt);
}

// Bitmap form: the same rank value over the row's selected blocks (a block
// is selected once, so the count is exact).
__global__ __launch_bounds__(256) void unit_work_bitmap_kernel(OrderParams p) {
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= p.n_units) return;
  const int qb = u % p.NQ;
  const int bh = u / p.NQ;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int64_t row = (int64_t)b * p.meta_sb + (int64_t)h * p.meta_sh + qb;
  const int8_t* mrow = p.mask + row * p.NK;
  long long w = 0, ps = 0, cnt = 0;
  for (int kb = lane; kb < p.NK; kb += 64) {
    if (mrow[kb] != 0) {
      w += p.vbs ? clampi(p.vbs[kb], 0, p.block) : p.block;
      ps += kb;
      cnt += 1;
    }
  }
  store_rank(p, u, lane, w, ps, cnt);
}

// One workgroup per (b, h): the keys ((2^32 - 1 - work) << 32 | qb) are
// distinct, so the position of q-block qb in the order is the number of
// keys below its own; every thread ranks its keys against all NQ keys in
// LDS (each step reads one key that every lane reads: a broadcast).
constexpr int SORT_THREADS = 1024;
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
static_assert(BSA_MAX_ORDER_QBLOCKS % SORT_THREADS == 0, "keys per thread");

__global__ __launch_bounds__(SORT_THREADS) void unit_sort_kernel(OrderParams p) {
  extern __shared__ __attribute__((aligned(16))) uint64_t keys[];
  int32_t* ord = p.order + (int64_t)blockIdx.x * p.NQ;
  const int n = p.NQ;
  uint64_t mine[BSA_MAX_ORDER_QBLOCKS / SORT_THREADS];
#pragma unroll
  for (int t = 0; t < BSA_MAX_ORDER_QBLOCKS / SORT_THREADS; ++t) {
    const int i = threadIdx.x + t * SORT_THREADS;
    if (i < n) {
      mine[t] = ((uint64_t)(0xFFFFFFFFu - (uint32_t)ord[i]) << 32) | (uint32_t)i;
      keys[i] = mine[t];
    }
  }
  __syncthreads();  // every work value is read before any position is written
#pragma unroll
  for (int t = 0; t < BSA_MAX_ORDER_QBLOCKS / SORT_THREADS; ++t) {
    const int i = threadIdx.x + t * SORT_THREADS;
    if (i < n) {
      // two keys per 16-byte LDS read, several reads in flight
      int rank = 0;
      int j = 0;
#pragma unroll 4
      for (; j + 1 < n; j += 2) {
        const u64x2 kk = *(const u64x2*)(keys + j);
        rank += (kk.x < mine[t] ? 1 : 0) + (kk.y < mine[t] ? 1 : 0);
      }
      if (j < n) rank += keys[j] < mine[t] ? 1 : 0;
      ord[rank] = (int32_t)(uint32_t)mine[t];
    }
  }
}

}  // namespace

// Library-internal (not part of the C ABI): replaces each of `groups`
// consecutive runs of `n` work values in `order` by the permutation of its
// indices in decreasing work, ties by index (the rank kernel above);
// n <= BSA_MAX_ORDER_QBLOCKS.  Used for the backward pass's units.
__attribute__((visibility("hidden"))) bsa_status bsa_rank_runs(int32_t* order,
                                                                int32_t groups,
                                                                int32_t n,
                                                                hipStream_t stream) {
  OrderParams p{};
  p.order = order;
  p.NQ = n;
  hipLaunchKernelGGL(unit_sort_kernel, dim3((unsigned)groups), dim3(SORT_THREADS),
                     (size_t)n * sizeof(uint64_t), stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

namespace {

// Checks shared by both forms (meta_ok: the form's own metadata sizes are
// valid); fills the sizes of p.
bsa_status order_setup(OrderParams& p, bool meta_ok, int64_t meta_stride_b,
                       int64_t meta_stride_h, const int32_t* vbs, int32_t* order,
                       int32_t B, int32_t H, int32_t S, int32_t Sk, int32_t block) {
  if (!order) return BSA_ERR_NULL;
  if (B <= 0 || H <= 0 || S <= 0 || Sk <= 0 || block <= 0) return BSA_ERR_SHAPE;
  if (S % block != 0 || Sk % block != 0) return BSA_ERR_SHAPE;
  if (!meta_ok || meta_stride_b < 0 || meta_stride_h < 0) return BSA_ERR_SHAPE;
  if (block != 64 && block != 128) return BSA_ERR_UNSUPPORTED;
  const int NQ = S / block;
  if (NQ > BSA_MAX_ORDER_QBLOCKS || Sk / block > BSA_MAX_KEY_BLOCKS)
    return BSA_ERR_UNSUPPORTED;
  const int64_t units = (int64_t)B * H * NQ;
  if (units > INT32_MAX) return BSA_ERR_UNSUPPORTED;
  p.meta_sb = meta_stride_b;
  p.meta_sh = meta_stride_h;
  p.vbs = vbs;
  p.order = order;
  p.H = H;
  p.NQ = NQ;
  p.NK = Sk / block;
  p.block = block;
  p.n_units = (int32_t)units;
  return BSA_OK;
}

template <typename WorkKernel>
bsa_status order_launch(WorkKernel work, const OrderParams& p, int32_t BH,
                        hipStream_t s) {
  hipLaunchKernelGGL(work, dim3((unsigned)((p.n_units + 3) / 4)), dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP;
  hipLaunchKernelGGL(unit_sort_kernel, dim3((unsigned)BH), dim3(SORT_THREADS),
                     (size_t)p.NQ * sizeof(uint64_t), s, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace

extern "C" bsa_status bsa_unit_order_lut(const int32_t* q2k_idx, const int32_t* q2k_num,
                                         int32_t max_kv, int64_t meta_stride_b,
                                         int64_t meta_stride_h,
                                         const int32_t* variable_block_sizes,
                                         int32_t* order, int32_t B, int32_t H, int32_t S,
                                         int32_t Sk, int32_t block, void* stream) {
  if (!q2k_idx || !q2k_num) return BSA_ERR_NULL;
  OrderParams p{};
  bsa_status st = order_setup(p, max_kv >= 1, meta_stride_b, meta_stride_h,
                              variable_block_sizes, order, B, H, S, Sk, block);
  if (st != BSA_OK) return st;
  p.idx = q2k_idx;
  p.num = q2k_num;
  p.max_kv = max_kv;
  return order_launch(unit_work_kernel, p, B * H, (hipStream_t)stream);
}

extern "C" bsa_status bsa_unit_order_bitmap(const int8_t* mask, int64_t mask_stride_b,
                                            int64_t mask_stride_h,
                                            const int32_t* variable_block_sizes,
                                            int32_t* order, int32_t B, int32_t H,
                                            int32_t S, int32_t Sk, int32_t block,
                                            void* stream) {
  if (!mask) return BSA_ERR_NULL;
  OrderParams p{};
  bsa_status st = order_setup(p, true, mask_stride_b, mask_stride_h,
                              variable_block_sizes, order, B, H, S, Sk, block);
  if (st != BSA_OK) return st;
  p.mask = mask;
  return order_launch(unit_work_bitmap_kernel, p, B * H, (hipStream_t)stream);
}
