// Device-side check of the paged-cache indices: every entry of block_table that
// a request reads (columns 0 .. ceil(cache_seqlens[b] / 64) - 1) must name a
// page of the cache, and every length must lie in [0, 64 * max_pages_per_seq].
// The decode kernels take both on trust (an entry out of range reads outside
// the cache), so this is the opt-in debug path: mla_check_paged_inputs runs
// it explicitly, and with MLA_DEBUG set the decode entry points run it before
// their own launches and return an error instead of launching.  Errors come
// back as a status and a message, never as a trap or an exit: page "FlashMLA:
// 高性能GPU注意力机制计算库 文件结构分析", section "火辣点评：FlashMLA的类设计",
// criticises the print-and-exit handling of bad input.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mla_api_util.h"
#include "mla_internal.h"

// The first violation found, as (request << 32) | (column + 1), column + 1 = 0
// for a bad length; all ones when there is none.  One copy per GPU.
static __device__ unsigned long long check_first[1];

namespace mla {

constexpr int kCheckThreads = 256;

__global__ void check_reset_kernel(unsigned long long* first) { first[0] = ~0ull; }

// One workgroup per request.
__global__ __launch_bounds__(kCheckThreads) void check_paged_kernel(const int32_t* __restrict__ block_table,
                                                                    int64_t bt_stride,
                                                                    const int32_t* __restrict__ seqlens,
                                                                    int max_pages, int num_pages,
                                                                    unsigned long long* first) {
  const int b = blockIdx.x;
  const int n = seqlens[b];
  const unsigned long long row = (unsigned long long)b << 32;
  if (n < 0 || (long long)n > 64LL * max_pages) {
    if (threadIdx.x == 0) atomicMin(first, row);
    return;
  }
  const int used = (n + 63) / 64;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  for (int j = threadIdx.x; j < used; j += kCheckThreads) {
    const int v = bt[j];
    if (v < 0 || v >= num_pages) atomicMin(first, row | (unsigned long long)(j + 1));
  }
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_check_mu;               // one check at a time: they share check_first
void* g_first_ptr[kMaxDevices];      // device address of check_first, per device

}  // namespace

bool debug_checks_enabled() {
  const char* v = std::getenv("MLA_DEBUG");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

mla_status check_paged_inputs(const int32_t* block_table, int64_t bt_stride, const int32_t* seqlens, int batch,
                              int max_pages, int num_pages, hipStream_t stream) {
  using api::fail;
  using api::hip_fail;
  if (!block_table || !seqlens) return fail(MLA_ERROR_INVALID_VALUE, "block_table and cache_seqlens must not be NULL");
  if (!api::aligned(block_table, 4) || !api::aligned(seqlens, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "block_table and cache_seqlens must be 4-byte aligned");
  if (batch <= 0 || max_pages <= 0 || num_pages <= 0)
    return fail(MLA_ERROR_INVALID_VALUE, "batch, max_pages_per_seq and num_pages must be positive");
  if (bt_stride < max_pages)
    return fail(MLA_ERROR_INVALID_VALUE, "bt_stride (%lld) < max_pages_per_seq (%d)", (long long)bt_stride, max_pages);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERROR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_check_mu);
  if (!g_first_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(check_first));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the check result");
    if (!ptr) return fail(MLA_ERROR_HIP, "hipGetSymbolAddress returned NULL for the check result");
    g_first_ptr[dev] = ptr;
  }
  auto* first = static_cast<unsigned long long*>(g_first_ptr[dev]);
  hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(1), 0, stream, first);
  hipLaunchKernelGGL(check_paged_kernel, dim3(batch), dim3(kCheckThreads), 0, stream, block_table, bt_stride,
                     seqlens, max_pages, num_pages, first);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "input check launch");
  unsigned long long found = 0;
  e = hipMemcpyAsync(&found, first, sizeof(found), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "input check readback");
  if (found == ~0ull) return MLA_SUCCESS;
  const int b = (int)(found >> 32);
  const int col = (int)(found & 0xffffffffu) - 1;
  int32_t value = 0;
  const int32_t* src = col < 0 ? seqlens + b : block_table + (int64_t)b * bt_stride + col;
  e = hipMemcpyAsync(&value, src, sizeof(value), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "input check readback");
  if (col < 0)
    return fail(MLA_ERROR_INVALID_VALUE, "cache_seqlens[%d] = %d lies outside [0, %lld] (64 * max_pages_per_seq)", b,
                value, 64LL * max_pages);
  return fail(MLA_ERROR_INVALID_VALUE, "block_table[%d][%d] = %d lies outside [0, %d) (num_pages)", b, col, value,
              num_pages);
}

}  // namespace mla

extern "C" mla_status mla_check_paged_inputs(const int32_t* block_table, int64_t bt_stride,
                                             const int32_t* cache_seqlens, int batch, int max_pages_per_seq,
                                             int num_pages, hipStream_t stream) {
  const mla_status st = mla::check_paged_inputs(block_table, bt_stride, cache_seqlens, batch, max_pages_per_seq,
                                                num_pages, stream);
  return st == MLA_SUCCESS ? mla::api::ok() : st;
}
