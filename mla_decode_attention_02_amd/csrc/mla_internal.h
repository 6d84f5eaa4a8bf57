// Launchers shared between the C ABI (mla_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeParams;
struct MergeParams;
struct MhaParams;

// Split requests cut into at most this many pieces are merged inside the
// split-KV kernel on the fused path.
constexpr int kFusedMaxPieces = 4;

// Split-KV attention, 64-row tiles: grid (num_parts, m_blocks), 512 threads.
// dtype 0 = bf16, 1 = fp16.
hipError_t launch_splitkv_wide(const DecodeParams& p, int dtype, int m_blocks, hipStream_t st);
// Split-KV attention, one tile of up to 16 rows: grid (num_parts), 256 threads.
hipError_t launch_splitkv_narrow(const DecodeParams& p, int dtype, hipStream_t st);
// The same over an fp8 e4m3 cache (bf16 q): grid (num_parts), 256 threads.
hipError_t launch_splitkv_fp8(const DecodeParams& p, hipStream_t st);
// 64-row tiles over an fp8 e4m3 cache (bf16 q): grid (num_parts, m_blocks), 512 threads.
hipError_t launch_splitkv_wide_fp8(const DecodeParams& p, int m_blocks, hipStream_t st);
// Merge of split pieces: grid (batch, ceil(rows / 4), 2 column halves), 256 threads.
hipError_t launch_combine(const DecodeParams& p, int dtype, hipStream_t st);
// Merge of context-parallel shards: grid (batch, ceil(rows / 4)), 256 threads.
hipError_t launch_merge(const MergeParams& m, int dtype, hipStream_t st);
// Tile schedule: one workgroup.  The units of work are `units` = batch * rep
// entries, unit u having length seqlens[u / rep] (rep = 1 for MLA requests,
// h_kv for the (request, KV head) units of the MHA path).
hipError_t launch_metadata(const int32_t* seqlens, int units, int rep, int num_parts, int fixed_overhead,
                           int32_t* sched, int32_t* split_offsets, hipStream_t st);
// Paged MHA/GQA split-KV attention: grid (num_parts, ceil(rows / 64)), 256
// threads.  head_dim 64, 128 or 256.
hipError_t launch_mha_splitkv(const MhaParams& p, int dtype, int head_dim, hipStream_t st);
// Merge of the MHA path's split pieces: grid (units, ceil(rows / 4)), 256 threads.
hipError_t launch_mha_combine(const MhaParams& p, int dtype, int head_dim, hipStream_t st);

}  // namespace mla
