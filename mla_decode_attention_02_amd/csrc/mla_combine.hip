// Merge of split-KV pieces by their log-sum-exp (page "FlashMLA 在 Hopper GPU
// 上的 MHA 内核调度优化解析", section "辅助优化：可编程依赖启动与瓦片调度": the
// combine kernel that follows splitkv_mla).  For a request cut into pieces k
// with normalised partial outputs O_k and LSE_k:
//   LSE = log sum_k exp(LSE_k),   O = sum_k exp(LSE_k - LSE) * O_k.
// One wave per query row; each lane owns 8 of the 512 columns.  Requests with
// no cached token get O = 0 and LSE = -inf; whole (unsplit) requests were
// already written by the split-KV kernel and are skipped.
#include "mla_common.hpp"
#include "mla_internal.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + wave;
  if (row >= p.rows) return;
  const int s0 = p.split_offsets[b];
  const int ns = p.split_offsets[b + 1] - s0;
  if (ns == 1) return;
  const int tok = row / p.h_q;
  const int head = row - tok * p.h_q;
  T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + lane * 8;
  float* lse_dst = p.lse + (int64_t)b * p.rows + row;

  float mx = -INFINITY;
  for (int k = 0; k < ns; ++k) mx = fmaxf(mx, p.part_lse[(int64_t)(s0 + k) * p.rows + row]);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int k = 0; k < ns; ++k)
      sum += __builtin_amdgcn_exp2f((p.part_lse[(int64_t)(s0 + k) * p.rows + row] - mx) * kLog2e);
    L = mx + __logf(sum);
    for (int k = 0; k < ns; ++k) {
      const int64_t slot = s0 + k;
      const float w = __builtin_amdgcn_exp2f((p.part_lse[slot * p.rows + row] - L) * kLog2e);
      const float* src = p.part_o + (slot * p.rows + row) * kDV + lane * 8;
      acc0 += w * *(const f32x4*)src;
      acc1 += w * *(const f32x4*)(src + 4);
    }
  }
  u32x4 wv = {Dt<T>::pack2(acc0[0], acc0[1]), Dt<T>::pack2(acc0[2], acc0[3]),
              Dt<T>::pack2(acc1[0], acc1[1]), Dt<T>::pack2(acc1[2], acc1[3])};
  *(u32x4*)dst = wv;
  if (lane == 0) *lse_dst = L;
}

hipError_t launch_combine(const DecodeParams& p, int dtype, hipStream_t st) {
  dim3 grid(p.batch, (p.rows + 3) / 4);
  if (dtype == 0) hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(combine_kernel<_Float16>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
