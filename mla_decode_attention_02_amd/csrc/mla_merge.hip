// Merge of the results of several shards of the same requests (context
// parallelism: each GPU holds a contiguous range of a request's cached tokens
// and runs the decode on it).  The identity is the one the combine kernel
// applies to the pieces of a split request (page "FlashMLA 在 Hopper GPU 上的 MHA
// 内核调度优化解析", section "辅助优化：可编程依赖启动与瓦片调度": partial results
// merged by their LSE): with shard outputs O_r (normalised, in the output
// dtype) and LSE_r,
//   LSE = log sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) * O_r,
// and O = 0, LSE = -inf when no shard saw a key.  One wave per query row; each
// lane owns 8 of the 512 columns (one 16-byte load per shard); the lanes load
// the shards' LSEs together and eight shards' outputs are loaded at a time.
#include "mla_common.hpp"
#include "mla_internal.h"

namespace mla {

namespace {

__device__ __forceinline__ float wmax(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}

__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  return x;
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams m) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + wave;
  const int rows = m.s_q * m.h_q;
  if (row >= rows) return;
  const int tok = row / m.h_q;
  const int head = row - tok * m.h_q;
  const int ns = m.num_shards;
  const int64_t src0 = b * m.p_s1 + tok * m.p_s2 + head * m.p_s3 + lane * 8;   // elements
  const int64_t lse0 = (int64_t)b * rows + row;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  float mx = -INFINITY;
  for (int k = lane; k < ns; k += 64) mx = fmaxf(mx, m.part_lse[k * m.lse_s + lse0]);
  mx = wmax(mx);
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int k = lane; k < ns; k += 64) sum += __builtin_amdgcn_exp2f((m.part_lse[k * m.lse_s + lse0] - mx) * kLog2e);
    L = mx + __logf(wsum(sum));
    for (int r0 = 0; r0 < ns; r0 += 64) {
      const int n = min(64, ns - r0);
      // weight of shard r0 + lane, exp(LSE_r - LSE) (0 past n), broadcast below
      const float lk = lane < n ? m.part_lse[(r0 + lane) * m.lse_s + lse0] : -INFINITY;
      const float w = __builtin_amdgcn_exp2f((lk - L) * kLog2e);
      for (int j = 0; j < n; j += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = j + u < n ? *(const u32x4*)((const T*)m.part_out + (int64_t)(r0 + j + u) * m.p_s0 + src0)
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float x, y;
            Dt<T>::unpack2(v[u][q], x, y);
            acc[2 * q] += wu * x;
            acc[2 * q + 1] += wu * y;
          }
        }
      }
    }
  }
  T* dst = (T*)m.out + b * m.o_s0 + tok * m.o_s1 + head * m.o_s2 + lane * 8;
  *(u32x4*)dst = u32x4{Dt<T>::pack2(acc[0], acc[1]), Dt<T>::pack2(acc[2], acc[3]), Dt<T>::pack2(acc[4], acc[5]),
                       Dt<T>::pack2(acc[6], acc[7])};
  if (lane == 0) m.lse[lse0] = L;
}

hipError_t launch_merge(const MergeParams& m, int dtype, hipStream_t st) {
  dim3 grid(m.batch, (m.s_q * m.h_q + 3) / 4);
  if (dtype == 0) hipLaunchKernelGGL(merge_kernel<__bf16>, grid, dim3(256), 0, st, m);
  else hipLaunchKernelGGL(merge_kernel<_Float16>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace mla
