// Merge of split-KV pieces by their log-sum-exp (page "FlashMLA 在 Hopper GPU
// 上的 MHA 内核调度优化解析", section "辅助优化：可编程依赖启动与瓦片调度": the
// combine kernel that follows splitkv_mla).  For a request cut into pieces k
// with normalised partial outputs O_k and LSE_k:
//   LSE = log sum_k exp(LSE_k),   O = sum_k exp(LSE_k - LSE) * O_k.
// One wave per query row, or per half row when rows are few; each lane owns 8
// or 4 columns.
// The lanes load the pieces' LSEs together (lane k holds piece k of a group of
// 64) and reduce them across the wave, while the first eight pieces' data loads
// are already in flight; the weighted sum keeps eight pieces' loads in flight
// per lane (sixteen with half rows: the next eight are issued before the
// current eight are summed), so a request cut into many pieces is not a chain
// of dependent memory round trips.  Requests with no cached token get
// O = 0 and LSE = -inf; whole (unsplit) requests, and split requests the
// split-KV kernel merged itself (at most fuse_max pieces), are skipped.
#include "mla_common.hpp"
#include "mla_sched.hpp"
#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
  return x;
}

// kCh = 16-byte column chunks per lane and piece: 1 (a wave covers half of
// the 512 columns) or 2 (the whole row, chunks 256 floats apart).  Pieces are
// loaded kB at a time: 8 with half rows (few rows, so few waves, each with
// many pieces to hide), 4 with whole rows, which keeps a wave within 64
// registers so that eight waves share a SIMD and a launch of many rows runs
// in one round.
template <typename T, int kCh>
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
  constexpr int kB = kCh == 1 ? 8 : 4;
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + wave;
  const int col = blockIdx.z * 256 + lane * 4;
  if (row >= p.rows) return;
  int s0, ns;
  if (p.split_offsets) {
    s0 = ldu(p.split_offsets + b);
    ns = ldu(p.split_offsets + b + 1) - s0;
  } else {
    // the split-KV kernel recorded them, for every request with a page
    const int n = ldu(p.seqlens + b);
    s0 = ldu(p.req_slots + 2 * b);
    const int rec_ns = ldu(p.req_slots + 2 * b + 1);
    ns = n > 0 ? rec_ns : 0;
  }
  if (ns == 1 || (ns > 1 && ns <= p.fuse_max)) return;   // whole, or merged by the split-KV kernel
  const float* lse_k = p.part_lse + (int64_t)s0 * p.rows + row;   // stride p.rows per piece

  const float* src = p.part_o + ((int64_t)s0 * p.rows + row) * kDV + col;
  const int64_t piece = (int64_t)p.rows * kDV;                      // floats between pieces
  f32x4 acc[kCh];
#pragma unroll
  for (int h = 0; h < kCh; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  auto load_batch = [&](f32x4 (&v)[kB][kCh], int k0, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kB; ++u)
#pragma unroll
      for (int h = 0; h < kCh; ++h)
        v[u][h] = k0 + u < n ? *(const f32x4*)(src + (k0 + u) * piece + h * 256) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto acc_batch = [&](const f32x4 (&v)[kB][kCh], float w, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j0 + u));
#pragma unroll
      for (int h = 0; h < kCh; ++h) acc[h] += wu * v[u][h];
    }
  };
  if (ns <= 64) {
    // the first eight pieces' data loads go out together with the LSE loads;
    // with half rows per wave (few rows, so typically many pieces each) the
    // next eight pieces' loads are issued before the current eight are summed
    f32x4 v[kCh == 1 ? 2 : 1][kB][kCh];
    load_batch(v[0], 0, ns);
    const float lk = lane < ns ? lse_k[(int64_t)lane * p.rows] : -INFINITY;
    const float mx = wave_max(lk);
    if (mx != -INFINITY) {
      const float e = lane < ns ? __builtin_amdgcn_exp2f((lk - mx) * kLog2e) : 0.f;
      const float sum = wave_sum(e);
      L = mx + __logf(sum);
      const float w = e / sum;                                      // exp(LSE_k - LSE)
      if constexpr (kCh == 1) {
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
          if (gi * kB >= ns) break;
          if (gi * kB + kB < ns) load_batch(v[(gi + 1) & 1], gi * kB + kB, ns);
          acc_batch(v[gi & 1], w, gi * kB);
        }
      } else {
        acc_batch(v[0], w, 0);
        for (int j = kB; j < ns; j += kB) {
          load_batch(v[0], j, ns);
          acc_batch(v[0], w, j);
        }
      }
    }
  } else {
    // more than 64 pieces: the LSEs are reduced in groups of 64
    float mx = -INFINITY;
    for (int k = lane; k < ns; k += 64) mx = fmaxf(mx, lse_k[(int64_t)k * p.rows]);
    mx = wave_max(mx);
    if (mx != -INFINITY) {
      float sum = 0.f;
      for (int k = lane; k < ns; k += 64) sum += __builtin_amdgcn_exp2f((lse_k[(int64_t)k * p.rows] - mx) * kLog2e);
      sum = wave_sum(sum);
      L = mx + __logf(sum);
      for (int k0 = 0; k0 < ns; k0 += 64) {
        const int kl = k0 + lane;
        const float w = kl < ns ? __builtin_amdgcn_exp2f((lse_k[(int64_t)kl * p.rows] - L) * kLog2e) : 0.f;
        const int n = min(64, ns - k0);
        for (int j = 0; j < n; j += kB) {
          f32x4 v[kB][kCh];
#pragma unroll
          for (int u = 0; u < kB; ++u)
#pragma unroll
            for (int h = 0; h < kCh; ++h)
              v[u][h] = j + u < n ? *(const f32x4*)(src + (k0 + j + u) * piece + h * 256) : f32x4{0.f, 0.f, 0.f, 0.f};
          acc_batch(v, w, j);
        }
      }
    }
  }
  const int tok = row / p.h_q;
  const int head = row - tok * p.h_q;
  T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + col;
#pragma unroll
  for (int h = 0; h < kCh; ++h)
    *(u32x2*)(dst + h * 256) = u32x2{Dt<T>::pack2(acc[h][0], acc[h][1]), Dt<T>::pack2(acc[h][2], acc[h][3])};
  if (blockIdx.z == 0 && lane == 0) p.lse[(int64_t)b * p.rows + row] = L;
}

hipError_t launch_combine(const DecodeParams& p, int dtype, hipStream_t st) {
  // whole rows per wave when there are enough rows to fill the chip, else
  // half rows (twice the waves)
  const bool whole = (int64_t)p.batch * p.rows >= 4096;
  dim3 grid(p.batch, (p.rows + 3) / 4, whole ? 1 : 2);
  if (dtype == 0) {
    if (whole) hipLaunchKernelGGL((combine_kernel<__bf16, 2>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((combine_kernel<__bf16, 1>), grid, dim3(256), 0, st, p);
  } else {
    if (whole) hipLaunchKernelGGL((combine_kernel<_Float16, 2>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((combine_kernel<_Float16, 1>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mla
