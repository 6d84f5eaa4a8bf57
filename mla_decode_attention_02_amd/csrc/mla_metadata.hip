// Split-KV tile scheduler (page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析",
// section "6. SM资源调度优化"): the work of all requests, in 64-token pages, is
// spread over num_parts partitions with a per-partition quota of
// ceil(total / num_parts) + F, where every piece of a request also costs the
// fixed overhead F.  Partitions are filled greedily in request order; a request
// that does not fit the remaining budget is cut after (budget - F) pages when
// that is positive.  The schedule is a few hundred integer steps, so a single
// lane builds it; the rest of the workgroup only computes the total cost.
#include "mla_common.hpp"
#include "mla_internal.h"

namespace mla {

__global__ __launch_bounds__(256) void metadata_kernel(const int32_t* __restrict__ seqlens, int batch,
                                                       int num_parts, int F, int32_t* __restrict__ sched,
                                                       int32_t* __restrict__ split_offsets) {
  __shared__ long long partial[256];
  const int tid = threadIdx.x;
  long long acc = 0;
  for (int b = tid; b < batch; b += blockDim.x) {
    const int pages = (seqlens[b] + kPage - 1) / kPage;
    if (pages > 0) acc += pages + F;
  }
  partial[tid] = acc;
  for (int b = tid; b < batch; b += blockDim.x) split_offsets[b + 1] = 0;
  __syncthreads();
  if (tid != 0) return;
  long long total = 0;
  for (int i = 0; i < (int)blockDim.x; ++i) total += partial[i];
  const long long quota = (total + num_parts - 1) / num_parts + F;

  int b = 0, pos = 0;   // next request, next page within it
  for (int part = 0; part < num_parts; ++part) {
    long long budget = quota;
    int nchunks = 0, b0 = 0, p0 = 0, s0 = 0, b1 = -1, p1 = 0;
    while (b < batch) {
      const int pages = (seqlens[b] + kPage - 1) / kPage;
      if (pages == 0) { ++b; pos = 0; continue; }
      const long long need = (long long)(pages - pos) + F;
      int lo = pos, hi;
      bool done;
      if (need <= budget) {
        hi = pages;
        budget -= need;
        done = true;
      } else {
        const long long take = budget - F;
        if (take <= 0) break;
        hi = pos + (int)take;
        done = false;
      }
      if (nchunks == 0) { b0 = b; p0 = lo; s0 = split_offsets[b + 1]; }
      b1 = b; p1 = hi;
      split_offsets[b + 1] += 1;
      ++nchunks;
      if (done) { ++b; pos = 0; } else { pos = hi; break; }
    }
    int32_t* row = sched + part * 8;
    if (nchunks == 0) {
      row[0] = 0; row[1] = 0; row[2] = -1; row[3] = 0; row[4] = 0; row[5] = 0;
    } else {
      row[0] = b0; row[1] = p0; row[2] = b1; row[3] = p1; row[4] = s0; row[5] = nchunks;
    }
    row[6] = 0; row[7] = 0;
  }
  split_offsets[0] = 0;
  for (int i = 0; i < batch; ++i) split_offsets[i + 1] += split_offsets[i];
}

hipError_t launch_metadata(const int32_t* seqlens, int batch, int num_parts, int fixed_overhead,
                           int32_t* sched, int32_t* split_offsets, hipStream_t st) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(256), 0, st, seqlens, batch, num_parts,
                     fixed_overhead, sched, split_offsets);
  return hipGetLastError();
}

}  // namespace mla
