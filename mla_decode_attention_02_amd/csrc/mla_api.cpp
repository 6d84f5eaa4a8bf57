// C ABI of the paged MLA decode library: argument checks, launch geometry and
// dispatch.  All computation happens in the kernels of mla_splitkv.hip,
// mla_combine.hip and mla_metadata.hip; this file never touches tensor data.
//
// Errors are reported as status codes with a per-thread message instead of the
// print-and-exit(1) handling criticised on page "FlashMLA: 高性能GPU注意力机制计算库
// 文件结构分析", section "火辣点评：FlashMLA的类设计".
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/mla_decode.h"
#include "mla_api_util.h"
#include "mla_common.hpp"
#include "mla_internal.h"

static_assert(mla::kFusedMaxPieces == MLA_FUSED_MAX_PIECES, "fused-merge limit");

// Workspace of mla_decode_noalloc: one copy on every GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device array: kernels only ever see the device address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace mla {
namespace api {

namespace {
thread_local std::string g_error;
}

mla_status fail(mla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

mla_status ok() {
  g_error.clear();
  return MLA_SUCCESS;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERROR_HIP, "%s: %s", what, hipGetErrorString(e));
}

const char* last_error() { return g_error.c_str(); }

}  // namespace api
}  // namespace mla

namespace {

using mla::api::aligned;
using mla::api::fail;
using mla::api::hip_fail;
using mla::api::ok;
using mla::api::round256;

// Query-row tile: 16 rows when everything fits one MFMA tile, else 64.
int tile_rows(int rows) { return rows <= 16 ? 16 : 64; }

mla_status check_shape(int batch, int s_q, int h_q, int h_kv) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0)
    return fail(MLA_ERROR_INVALID_VALUE, "batch, s_q and h_q must be positive (got %d, %d, %d)", batch, s_q, h_q);
  if (h_kv != 1) return fail(MLA_ERROR_UNSUPPORTED, "only one latent KV head is supported (h_kv=%d)", h_kv);
  const long long rows = (long long)s_q * h_q;
  if (rows > 64LL * 65535) return fail(MLA_ERROR_INVALID_VALUE, "s_q*h_q=%lld exceeds %d", rows, 64 * 65535);
  if ((long long)batch > 2147483647LL / 8) return fail(MLA_ERROR_INVALID_VALUE, "batch too large");
  return MLA_SUCCESS;
}

// Workspace: the arrival counters of the fused merge [m_blocks, batch] int32
// first (their place depends on the shape only, not on num_parts), then each
// request's first piece slot and piece count [batch][2] int32 (written when
// the kernels derive the schedule themselves), then fp32 partial outputs
// [slots, rows, 512] and their LSEs [slots, rows]; each region starts on a
// 256-byte boundary.

size_t counters_bytes(int batch, int s_q, int h_q) {
  const int rows = s_q * h_q;
  const size_t m_blocks = (size_t)((rows + tile_rows(rows) - 1) / tile_rows(rows));
  return round256(m_blocks * (size_t)batch * sizeof(int32_t));
}

size_t req_slots_bytes(int batch) { return round256((size_t)batch * 2 * sizeof(int32_t)); }

size_t workspace_bytes(int batch, int s_q, int h_q, int num_parts) {
  const size_t slots = (size_t)batch + (size_t)num_parts;
  const size_t rows = (size_t)s_q * h_q;
  return counters_bytes(batch, s_q, h_q) + req_slots_bytes(batch) +
         round256(slots * rows * (mla::kDV + 1) * sizeof(float));
}

mla_status check_decode(const mla_decode_args* a) {
  if (!a) return fail(MLA_ERROR_INVALID_VALUE, "args is NULL");
  if (a->dtype != MLA_DTYPE_BF16 && a->dtype != MLA_DTYPE_FP16)
    return fail(MLA_ERROR_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", a->dtype);
  if (a->d_k != MLA_D_K || a->d_v != MLA_D_V)
    return fail(MLA_ERROR_UNSUPPORTED, "only d_k=576, d_v=512 are supported (got %d, %d)", a->d_k, a->d_v);
  if (a->page_size != MLA_PAGE_SIZE)
    return fail(MLA_ERROR_UNSUPPORTED, "page_size must be 64 (got %d)", a->page_size);
  mla_status st = check_shape(a->batch, a->s_q, a->h_q, a->h_kv);
  if (st != MLA_SUCCESS) return st;
  if (a->kv_dtype != MLA_KV_SAME && a->kv_dtype != MLA_KV_FP8_E4M3 && a->kv_dtype != MLA_KV_FP8_E4M3_QK8)
    return fail(MLA_ERROR_UNSUPPORTED,
                "kv_dtype %d is not MLA_KV_SAME (0), MLA_KV_FP8_E4M3 (1) or MLA_KV_FP8_E4M3_QK8 (2)", a->kv_dtype);
  if (a->kv_dtype != MLA_KV_SAME && a->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERROR_UNSUPPORTED, "an fp8 cache needs dtype bf16");
  if (a->k_scale && !aligned(a->k_scale, 4)) return fail(MLA_ERROR_INVALID_VALUE, "k_scale must be 4-byte aligned");
  if (a->num_pages <= 0 || a->max_pages_per_seq <= 0 || a->num_parts <= 0)
    return fail(MLA_ERROR_INVALID_VALUE, "num_pages, max_pages_per_seq and num_parts must be positive");
  if (!a->q || !a->k_cache || !a->block_table || !a->cache_seqlens || !a->workspace || !a->out || !a->lse)
    return fail(MLA_ERROR_INVALID_VALUE, "a required pointer is NULL");
  if (!a->sched != !a->split_offsets)
    return fail(MLA_ERROR_INVALID_VALUE, "sched and split_offsets must both be given or both be NULL");
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->workspace, 16))
    return fail(MLA_ERROR_INVALID_VALUE, "q, out and workspace must be 16-byte aligned");
  if (!aligned(a->k_cache, a->kv_dtype != MLA_KV_SAME ? 8 : 16))
    return fail(MLA_ERROR_INVALID_VALUE, "k_cache must be 16-byte aligned (8 for an fp8 cache)");
  if (!aligned(a->lse, 4) || !aligned(a->block_table, 4) || !aligned(a->cache_seqlens, 4) ||
      !aligned(a->sched, 4) || !aligned(a->split_offsets, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "lse and the int32 arrays must be 4-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (a->q_stride[i] <= 0 || a->q_stride[i] % 8)
      return fail(MLA_ERROR_INVALID_VALUE, "q_stride[%d]=%lld must be a positive multiple of 8", i, (long long)a->q_stride[i]);
    if (a->out_stride[i] <= 0 || a->out_stride[i] % 8)
      return fail(MLA_ERROR_INVALID_VALUE, "out_stride[%d]=%lld must be a positive multiple of 8", i, (long long)a->out_stride[i]);
  }
  for (int i = 0; i < 2; ++i)
    if (a->k_stride[i] <= 0 || a->k_stride[i] % 8)
      return fail(MLA_ERROR_INVALID_VALUE, "k_stride[%d]=%lld must be a positive multiple of 8", i, (long long)a->k_stride[i]);
  if (a->k_stride[1] < MLA_D_K)
    return fail(MLA_ERROR_INVALID_VALUE, "k_stride[1]=%lld is smaller than a row (576)", (long long)a->k_stride[1]);
  if ((long long)a->k_stride[1] * 2 * (MLA_PAGE_SIZE - 1) + MLA_D_K * 2 > 2147483647LL)
    return fail(MLA_ERROR_INVALID_VALUE, "k_stride[1] too large");
  if (a->q_stride[2] < MLA_D_K || a->out_stride[2] < MLA_D_V)
    return fail(MLA_ERROR_INVALID_VALUE, "head strides must cover a row (q >= 576, out >= 512)");
  if (a->bt_stride < a->max_pages_per_seq)
    return fail(MLA_ERROR_INVALID_VALUE, "bt_stride (%lld) < max_pages_per_seq (%d)", (long long)a->bt_stride, a->max_pages_per_seq);
  if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f))
    return fail(MLA_ERROR_INVALID_VALUE, "softmax_scale must be finite and positive");
  if (a->causal != 0 && a->causal != 1) return fail(MLA_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  const size_t need = workspace_bytes(a->batch, a->s_q, a->h_q, a->num_parts);
  if (a->workspace_bytes < need)
    return fail(MLA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the %zu required",
                a->workspace_bytes, need);
  return MLA_SUCCESS;
}

mla::DecodeParams make_params(const mla_decode_args* a) {
  mla::DecodeParams p;
  p.q = a->q;
  p.q_s0 = a->q_stride[0]; p.q_s1 = a->q_stride[1]; p.q_s2 = a->q_stride[2];
  p.k = a->k_cache;
  p.k_s0 = a->k_stride[0]; p.k_s1 = a->k_stride[1];
  p.kv_fp8 = a->kv_dtype != MLA_KV_SAME;
  p.qk8 = a->kv_dtype == MLA_KV_FP8_E4M3_QK8;
  p.k_scale = a->k_scale;
  p.block_table = a->block_table;
  p.bt_s = a->bt_stride;
  p.seqlens = a->cache_seqlens;
  p.sched = a->sched;
  p.split_offsets = a->split_offsets;
  p.sched_f = MLA_FIXED_OVERHEAD;
  p.batch = a->batch; p.s_q = a->s_q; p.h_q = a->h_q;
  p.rows = a->s_q * a->h_q;
  p.num_parts = a->num_parts;
  p.causal = a->causal;
  p.scale_log2 = a->softmax_scale * mla::kLog2e;
  p.out = a->out;
  p.o_s0 = a->out_stride[0]; p.o_s1 = a->out_stride[1]; p.o_s2 = a->out_stride[2];
  p.lse = a->lse;
  const size_t slots = (size_t)a->batch + (size_t)a->num_parts;
  p.counters = static_cast<int*>(a->workspace);
  char* ws = static_cast<char*>(a->workspace) + counters_bytes(a->batch, a->s_q, a->h_q);
  p.req_slots = reinterpret_cast<int*>(ws);
  p.part_o = reinterpret_cast<float*>(ws + req_slots_bytes(a->batch));
  p.part_lse = p.part_o + slots * (size_t)p.rows * mla::kDV;
  p.fuse_max = 0;
  return p;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return mla::api::last_error(); }

int mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status mla_get_metadata_shape(int num_cus, int batch, int s_q, int h_q, int h_kv, int* num_parts,
                                  int* sched_elems, int* split_offsets_elems) {
  mla_status st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_SUCCESS) return st;
  if (!num_parts || !sched_elems || !split_offsets_elems)
    return fail(MLA_ERROR_INVALID_VALUE, "output pointers must not be NULL");
  if (num_cus < 0) return fail(MLA_ERROR_INVALID_VALUE, "num_cus must be >= 0");
  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (num_cus <= 0) return fail(MLA_ERROR_HIP, "device reports %d compute units", num_cus);
  }
  const int rows = s_q * h_q;
  const int m_blocks = (rows + tile_rows(rows) - 1) / tile_rows(rows);
  int parts = num_cus / m_blocks;
  if (parts < 1) parts = 1;
  *num_parts = parts;
  *sched_elems = parts * MLA_SCHED_FIELDS;
  *split_offsets_elems = batch + 1;
  return ok();
}

mla_status mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                            int num_parts, int32_t* sched, int32_t* split_offsets, hipStream_t stream) {
  return mla_get_metadata_ex(cache_seqlens, batch, s_q, h_q, h_kv, num_parts, MLA_FIXED_OVERHEAD, sched,
                             split_offsets, stream);
}

mla_status mla_get_metadata_ex(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                               int num_parts, int fixed_overhead, int32_t* sched, int32_t* split_offsets,
                               hipStream_t stream) {
  mla_status st = check_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_SUCCESS) return st;
  if (num_parts <= 0) return fail(MLA_ERROR_INVALID_VALUE, "num_parts must be positive");
  if (fixed_overhead < 0 || fixed_overhead > 64)
    return fail(MLA_ERROR_INVALID_VALUE, "fixed_overhead must lie in [0, 64] (got %d)", fixed_overhead);
  if (!cache_seqlens || !sched || !split_offsets) return fail(MLA_ERROR_INVALID_VALUE, "NULL pointer");
  if (!aligned(cache_seqlens, 4) || !aligned(sched, 4) || !aligned(split_offsets, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "int32 arrays must be 4-byte aligned");
  hipError_t e = mla::launch_metadata(cache_seqlens, batch, 1, num_parts, fixed_overhead, sched,
                                      split_offsets, stream);
  if (e != hipSuccess) return hip_fail(e, "metadata launch");
  return ok();
}

mla_status mla_workspace_size(int batch, int s_q, int h_q, int num_parts, size_t* bytes) {
  if (!bytes) return fail(MLA_ERROR_INVALID_VALUE, "bytes is NULL");
  mla_status st = check_shape(batch, s_q, h_q, 1);
  if (st != MLA_SUCCESS) return st;
  if (num_parts <= 0) return fail(MLA_ERROR_INVALID_VALUE, "num_parts must be positive");
  *bytes = workspace_bytes(batch, s_q, h_q, num_parts);
  return ok();
}

namespace {

mla_status launch_splitkv(const mla_decode_args* args, const mla::DecodeParams& p, hipStream_t stream) {
  const int tile = tile_rows(p.rows);
  const int m_blocks = (p.rows + tile - 1) / tile;
  hipStream_t hs = stream;
  // up to 16 rows: the 16-row kernels (an fp8 cache, with either score
  // product, goes to the fp8 one); more: the 64-row kernels
  hipError_t e = tile == 16 ? mla::launch_splitkv_narrow(p, args->dtype, hs)
                 : p.kv_fp8 ? mla::launch_splitkv_wide_fp8(p, m_blocks, hs)
                            : mla::launch_splitkv_wide(p, args->dtype, m_blocks, hs);
  if (e != hipSuccess) return hip_fail(e, "split-KV launch");
  return ok();
}

mla_status launch_combine(const mla_decode_args* args, const mla::DecodeParams& p, hipStream_t stream) {
  hipError_t e = mla::launch_combine(p, args->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

// With MLA_DEBUG set: the device check of the paged-cache indices.
mla_status debug_check(const mla_decode_args* a, hipStream_t stream) {
  if (!mla::debug_checks_enabled()) return MLA_SUCCESS;
  return mla::check_paged_inputs(a->block_table, a->bt_stride, a->cache_seqlens, a->batch, a->max_pages_per_seq,
                                 a->num_pages, stream);
}

}  // namespace

mla_status mla_decode_splitkv(const mla_decode_args* args, hipStream_t stream) {
  mla_status st = check_decode(args);
  if (st == MLA_SUCCESS) st = debug_check(args, stream);
  if (st != MLA_SUCCESS) return st;
  return launch_splitkv(args, make_params(args), stream);
}

mla_status mla_decode_combine(const mla_decode_args* args, hipStream_t stream) {
  mla_status st = check_decode(args);
  if (st != MLA_SUCCESS) return st;
  return launch_combine(args, make_params(args), stream);
}

mla_status mla_decode(const mla_decode_args* args, hipStream_t stream) {
  mla_status st = mla_decode_splitkv(args, stream);
  if (st != MLA_SUCCESS) return st;
  return mla_decode_combine(args, stream);
}

mla_status mla_merge_partials(const mla_merge_args* a, hipStream_t stream) {
  if (!a) return fail(MLA_ERROR_INVALID_VALUE, "args is NULL");
  if (a->dtype != MLA_DTYPE_BF16 && a->dtype != MLA_DTYPE_FP16)
    return fail(MLA_ERROR_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", a->dtype);
  if (a->num_shards <= 0) return fail(MLA_ERROR_INVALID_VALUE, "num_shards must be positive");
  mla_status st = check_shape(a->batch, a->s_q, a->h_q, 1);
  if (st != MLA_SUCCESS) return st;
  if (!a->part_out || !a->part_lse || !a->out || !a->lse)
    return fail(MLA_ERROR_INVALID_VALUE, "a required pointer is NULL");
  if (!aligned(a->part_out, 16) || !aligned(a->out, 16))
    return fail(MLA_ERROR_INVALID_VALUE, "part_out and out must be 16-byte aligned");
  if (!aligned(a->part_lse, 4) || !aligned(a->lse, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "part_lse and lse must be 4-byte aligned");
  for (int i = 0; i < 4; ++i)
    if (a->part_out_stride[i] <= 0 || a->part_out_stride[i] % 8)
      return fail(MLA_ERROR_INVALID_VALUE, "part_out_stride[%d]=%lld must be a positive multiple of 8", i,
                  (long long)a->part_out_stride[i]);
  for (int i = 0; i < 3; ++i)
    if (a->out_stride[i] <= 0 || a->out_stride[i] % 8)
      return fail(MLA_ERROR_INVALID_VALUE, "out_stride[%d]=%lld must be a positive multiple of 8", i,
                  (long long)a->out_stride[i]);
  if (a->part_out_stride[3] < MLA_D_V || a->out_stride[2] < MLA_D_V)
    return fail(MLA_ERROR_INVALID_VALUE, "head strides must cover a row (>= 512)");
  const long long rows_total = (long long)a->batch * a->s_q * a->h_q;
  if (a->part_lse_stride < rows_total)
    return fail(MLA_ERROR_INVALID_VALUE, "part_lse_stride (%lld) is below batch*s_q*h_q (%lld)",
                (long long)a->part_lse_stride, rows_total);
  mla::MergeParams m;
  m.part_out = a->part_out;
  m.p_s0 = a->part_out_stride[0]; m.p_s1 = a->part_out_stride[1];
  m.p_s2 = a->part_out_stride[2]; m.p_s3 = a->part_out_stride[3];
  m.part_lse = a->part_lse;
  m.lse_s = a->part_lse_stride;
  m.num_shards = a->num_shards;
  m.batch = a->batch; m.s_q = a->s_q; m.h_q = a->h_q;
  m.out = a->out;
  m.o_s0 = a->out_stride[0]; m.o_s1 = a->out_stride[1]; m.o_s2 = a->out_stride[2];
  m.lse = a->lse;
  hipError_t e = mla::launch_merge(m, a->dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// This device's copy of `scratch`, looked up on the first call on the device.
mla_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERROR_UNSUPPORTED, "device %d is beyond the %d devices mla_decode_noalloc serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static workspace");
    if (!ptr) return fail(MLA_ERROR_HIP, "hipGetSymbolAddress returned NULL for the static workspace");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_SUCCESS;
}

}  // namespace

mla_status mla_decode_noalloc(const mla_decode_args* args, hipStream_t stream) {
  if (!args) return fail(MLA_ERROR_INVALID_VALUE, "args is NULL");
  mla_status st = check_shape(args->batch, args->s_q, args->h_q, args->h_kv);
  if (st != MLA_SUCCESS) return st;
  if (args->num_parts <= 0) return fail(MLA_ERROR_INVALID_VALUE, "num_parts must be positive");
  const size_t need = workspace_bytes(args->batch, args->s_q, args->h_q, args->num_parts);
  if (need > MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERROR_WORKSPACE_TOO_SMALL,
                "batch %d, s_q*h_q %d and num_parts %d need %zu bytes of workspace; the static workspace of "
                "mla_decode_noalloc holds %zu (use mla_decode with a caller workspace)",
                args->batch, args->s_q * args->h_q, args->num_parts, need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  // the host checks of mla_decode, against a placeholder for the workspace
  // (replaced by the device array below), before any HIP call
  mla_decode_args a = *args;
  a.workspace = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  a.workspace_bytes = MLA_NOALLOC_SCRATCH_BYTES;
  st = check_decode(&a);
  if (st == MLA_SUCCESS) st = debug_check(&a, stream);
  if (st != MLA_SUCCESS) return st;
  void* ptr = nullptr;
  st = scratch_on_current_device(&ptr);
  if (st != MLA_SUCCESS) return st;
  a.workspace = ptr;
  // the split-KV + combine pair of mla_decode: partial outputs only, no
  // counters (those belong to the fused path), nothing to clear first
  const mla::DecodeParams p = make_params(&a);
  st = launch_splitkv(&a, p, stream);
  if (st != MLA_SUCCESS) return st;
  return launch_combine(&a, p, stream);
}

mla_status mla_decode_fused(const mla_decode_args* args, hipStream_t stream) {
  mla_status st = check_decode(args);
  if (st == MLA_SUCCESS) st = debug_check(args, stream);
  if (st != MLA_SUCCESS) return st;
  mla::DecodeParams p = make_params(args);
  p.fuse_max = mla::kFusedMaxPieces;
  st = launch_splitkv(args, p, stream);
  if (st != MLA_SUCCESS) return st;
  return launch_combine(args, p, stream);
}

}  // extern "C"
