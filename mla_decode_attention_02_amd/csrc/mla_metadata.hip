// Split-KV tile scheduler (page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析",
// section "6. SM资源调度优化"): the work of all requests, in 64-token pages, is
// spread over num_parts partitions with a per-partition quota of
// ceil(total / num_parts) + F, where F is the fixed overhead every piece of a
// request costs.
//
// Assignment rule: a nonempty request b costs c_b = pages_b + F.  The costs are
// laid end to end in request order, request b starting at C_b with its F
// overhead units first, so page p of request b sits at position C_b + F + p.
// With T = sum of costs and W = ceil(T / num_parts), partition k takes the pages
// whose positions fall in [k W, (k+1) W).  A partition pays at most one F that
// lies outside its interval (a piece starting inside a request), so its cost
// stays within the quota W + F.
//
// Everything is data-parallel: one workgroup scans the costs into C (LDS, or
// split_offsets as scratch for very large batches), each thread then places one
// or more partitions with two binary searches over C, and a second scan turns
// the per-request piece counts into split_offsets.
#include "mla_common.hpp"
#include "mla_internal.h"

namespace mla {

constexpr int kMetaThreads = 256;
constexpr int kMetaWaves = kMetaThreads / 64;
constexpr int kMetaLdsBatch = 16384;   // requests whose start positions fit in LDS

__device__ __forceinline__ int pages_of(int n) { return (n + kPage - 1) / kPage; }

// Exclusive prefix sum of one value per thread across the workgroup.
__device__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kMetaWaves; ++w) {
    const int s = scratch[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// Largest request index b with C[b] <= pos (C[0] = 0 <= pos).  For pos < T this
// is the nonempty request whose cost interval holds pos.
__device__ __forceinline__ int find_request(const int* C, int batch, long long pos) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (C[mid] <= pos) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// `batch` counts units of work here; unit b has length seqlens[b / rep].
__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                                int rep, int num_parts, int F,
                                                                int32_t* __restrict__ sched,
                                                                int32_t* __restrict__ split_offsets) {
  __shared__ int scan_s[kMetaWaves];
  __shared__ int start_s[kMetaLdsBatch + 1];
  const int tid = threadIdx.x;
  const int per = (batch + kMetaThreads - 1) / kMetaThreads;
  const int lo = min(batch, tid * per);
  const int hi = min(batch, lo + per);
  // start positions: LDS when they fit, else split_offsets (overwritten at the end)
  int* C = batch <= kMetaLdsBatch ? start_s : split_offsets;

  // each thread parks the costs of its own requests in C, then turns them
  // into start positions in place: the lengths are read from memory once
  int local = 0;
  for (int b = lo; b < hi; ++b) {
    const int p = pages_of(seqlens[b / rep]);
    const int c = p > 0 ? p + F : 0;
    C[b] = c;
    local += c;
  }
  int total;
  const int first = block_exclusive_scan(local, scan_s, total);
  {
    int run = first;
    for (int b = lo; b < hi; ++b) {
      const int c = C[b];
      C[b] = run;
      run += c;
    }
    if (tid == 0) C[batch] = total;
  }
  __syncthreads();
  const int width = total > 0 ? (total + num_parts - 1) / num_parts : 1;

  // pieces per request: how many partitions its page positions touch.  While
  // C sits in LDS the lengths are not read again: a request costs
  // C[b+1] - C[b], its pages are that less F (empty requests cost 0).  With C
  // staged in split_offsets the last loop below overwrites it, so the lengths
  // are read again there.
  const bool c_in_lds = batch <= kMetaLdsBatch;
  auto cost_at = [&](int b) {
    if (c_in_lds) return C[b + 1] - C[b];
    const int p = pages_of(seqlens[b / rep]);
    return p > 0 ? p + F : 0;
  };
  auto pieces = [&](int start, int cost) {
    const int p = cost > 0 ? cost - F : 0;
    return p > 0 ? (start + F + p - 1) / width - (start + F) / width + 1 : 0;
  };
  int nsum = 0;
  {
    int run = first;
    for (int b = lo; b < hi; ++b) {
      const int c = cost_at(b);
      nsum += pieces(run, c);
      run += c;
    }
  }

  // partitions
  for (int k = tid; k < num_parts; k += kMetaThreads) {
    const long long s = (long long)k * width;
    const long long e = min((long long)total, s + width);
    int row[8] = {0, 0, -1, 0, 0, 0, 0, 0};
    if (s < total) {
      const int b0 = find_request(C, batch, s);
      const int c0 = C[b0];
      if ((long long)c0 + F < e) {
        const int p0 = s < (long long)c0 + F ? 0 : (int)(s - c0 - F);
        long long last = e - 1;
        int b1 = find_request(C, batch, last);
        if (last < (long long)C[b1] + F) {      // part ends inside b1's overhead
          last = (long long)C[b1] - 1;
          b1 = find_request(C, batch, last);
        }
        row[0] = b0;
        row[1] = p0;
        row[2] = b1;
        row[3] = (int)(last - C[b1] - F + 1);
        row[4] = k - (c0 + F) / width;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sched[k * 8 + i] = row[i];
  }

  int nall;
  const int sfirst = block_exclusive_scan(nsum, scan_s, nall);   // also orders the reads of C above
  {
    int run = sfirst, start = first;
    for (int b = lo; b < hi; ++b) {
      const int c = cost_at(b);        // C in LDS, or the length: never the entry overwritten here
      split_offsets[b] = run;
      run += pieces(start, c);
      start += c;
    }
    if (tid == 0) split_offsets[batch] = nall;
  }
}

hipError_t launch_metadata(const int32_t* seqlens, int units, int rep, int num_parts, int fixed_overhead,
                           int32_t* sched, int32_t* split_offsets, hipStream_t st) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMetaThreads), 0, st, seqlens, units, rep, num_parts,
                     fixed_overhead, sched, split_offsets);
  return hipGetLastError();
}

}  // namespace mla
