// Host-side helpers shared by the C ABI files (mla_api.cpp, mha_api.cpp): the
// per-thread error text behind mla_last_error() and small checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {
namespace api {

// Record a formatted message for mla_last_error() and return `st`.
mla_status fail(mla_status st, const char* fmt, ...);
// Clear the message and return MLA_SUCCESS.
mla_status ok();
// MLA_ERROR_HIP with the HIP error string.
mla_status hip_fail(hipError_t e, const char* what);
// The calling thread's message ("" if none).
const char* last_error();

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace api

// True when the environment variable MLA_DEBUG is set to anything but "" or
// "0": the decode entry points then check the paged-cache indices on the
// device before launching (synchronous, so not for graph capture).
bool debug_checks_enabled();
// The device check of block_table and cache_seqlens (mla_check.hip): waits
// for `stream`; MLA_ERROR_INVALID_VALUE naming the first bad entry.  Leaves
// the error text alone on success.
mla_status check_paged_inputs(const int32_t* block_table, int64_t bt_stride, const int32_t* seqlens, int batch,
                              int max_pages, int num_pages, hipStream_t stream);
}  // namespace mla
