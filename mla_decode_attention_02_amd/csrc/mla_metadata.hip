// Split-KV tile scheduler (page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析",
// section "6. SM资源调度优化"): the work of all requests, in 64-token pages, is
// spread over num_parts partitions with a per-partition quota of
// ceil(total / num_parts) + F, where F is the fixed overhead every piece of a
// request costs.
//
// Assignment rule: a nonempty request b costs c_b = pages_b + F.  The costs are
// laid end to end in request order, request b starting at C_b with
// F0 = floor(F / 2) overhead units, then its pages, then the other F - F0, so
// page p of request b sits at position C_b + F0 + p.  With T = sum of costs and
// W = ceil(T / num_parts), partition k takes the pages whose positions fall in
// [k W, (k+1) W).  Every piece costs F, but a partition's interval misses at
// most F0 of its first piece's overhead and F - F0 of its last one's, so its
// cost stays within the quota W + F; overhead on both sides of the pages makes
// a request cut in two split in the middle.
//
// The rule itself lives in mla_sched.hpp as wave-level functions, which the
// split-KV and combine kernels also evaluate in place when a call brings no
// schedule; this kernel writes their results out once per decode step for
// callers that reuse one schedule across layers.  Every wave is independent:
// wave k < num_parts writes partition k's row, the waves after it write
// split_offsets 64 entries at a time.
#include "mla_common.hpp"
#include "mla_internal.h"
#include "mla_sched.hpp"

namespace mla {

constexpr int kMetaThreads = 256;
constexpr int kMetaWaves = kMetaThreads / 64;

// `units` counts units of work here; unit u has length seqlens[u / rep].
__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(const int32_t* __restrict__ seqlens, int units,
                                                                int rep, int num_parts, int F,
                                                                int32_t* __restrict__ sched,
                                                                int32_t* __restrict__ split_offsets) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kMetaWaves + (threadIdx.x >> 6);
  if (w < num_parts) {
    const SchedRow r = sched_row(seqlens, units, rep, num_parts, F, w);
    const bool has = r.b1 >= r.b0;
    const int row[8] = {r.b0, r.p0, r.b1, r.p1, r.split0, 0, 0, 0};
    if (lane < 8) {
      int v = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) v = lane == i ? row[i] : v;
      sched[(int64_t)w * 8 + lane] = has ? v : (lane == 2 ? -1 : 0);
    }
  } else {
    const int u0 = (w - num_parts) * 64;
    if (u0 > units) return;                       // uniform over the wave
    int before, own;
    sched_slots(seqlens, units, rep, num_parts, F, u0, before, own);
    if (u0 + lane <= units) split_offsets[u0 + lane] = before;
  }
}

hipError_t launch_metadata(const int32_t* seqlens, int units, int rep, int num_parts, int fixed_overhead,
                           int32_t* sched, int32_t* split_offsets, hipStream_t st) {
  const long long waves = (long long)num_parts + (units + 1 + 63) / 64;
  const long long blocks = (waves + kMetaWaves - 1) / kMetaWaves;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(metadata_kernel, dim3((unsigned)blocks), dim3(kMetaThreads), 0, st, seqlens, units, rep,
                     num_parts, fixed_overhead, sched, split_offsets);
  return hipGetLastError();
}

}  // namespace mla
