// C ABI of the paged MHA/GQA decode path: argument checks, launch geometry
// and dispatch.  All computation happens in the kernels of mha_decode.hip and
// mla_metadata.hip; this file never touches tensor data.  Status codes and the
// per-thread error text are shared with the MLA entry points (mla_api.cpp).
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/mha_decode.h"
#include "mla_api_util.h"
#include "mla_common.hpp"
#include "mla_internal.h"

namespace {

using mla::api::aligned;
using mla::api::fail;
using mla::api::hip_fail;
using mla::api::ok;
using mla::api::round256;

constexpr int kRowBlock = 64;   // query rows per workgroup

mla_status check_mha_shape(int batch, int s_q, int h_q, int h_kv) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || h_kv <= 0)
    return fail(MLA_ERROR_INVALID_VALUE, "batch, s_q, h_q and h_kv must be positive (got %d, %d, %d, %d)", batch,
                s_q, h_q, h_kv);
  if (h_q % h_kv != 0) return fail(MLA_ERROR_INVALID_VALUE, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  const long long rows = (long long)s_q * (h_q / h_kv);
  if (rows > 4LL * 65535)   // the combine grid has one row of 4 query rows per y index
    return fail(MLA_ERROR_INVALID_VALUE, "s_q*h_q/h_kv=%lld exceeds %d", rows, 4 * 65535);
  if ((long long)batch * h_kv > 2147483647LL / 8) return fail(MLA_ERROR_INVALID_VALUE, "batch*h_kv too large");
  return MLA_SUCCESS;
}

size_t mha_workspace_bytes(int batch, int s_q, int h_q, int h_kv, int head_dim, int num_parts) {
  const size_t slots = (size_t)batch * h_kv + (size_t)num_parts;
  const size_t rows = (size_t)s_q * (h_q / h_kv);
  return round256(slots * rows * ((size_t)head_dim + 1) * sizeof(float));
}

mla_status check_mha(const mha_decode_args* a) {
  if (!a) return fail(MLA_ERROR_INVALID_VALUE, "args is NULL");
  if (a->dtype != MLA_DTYPE_BF16 && a->dtype != MLA_DTYPE_FP16)
    return fail(MLA_ERROR_UNSUPPORTED, "dtype %d is not bf16 (0) or fp16 (1)", a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(MLA_ERROR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
  if (a->page_size != MLA_PAGE_SIZE)
    return fail(MLA_ERROR_UNSUPPORTED, "page_size must be 64 (got %d)", a->page_size);
  mla_status st = check_mha_shape(a->batch, a->s_q, a->h_q, a->h_kv);
  if (st != MLA_SUCCESS) return st;
  if (a->num_pages <= 0 || a->max_pages_per_seq <= 0 || a->num_parts <= 0)
    return fail(MLA_ERROR_INVALID_VALUE, "num_pages, max_pages_per_seq and num_parts must be positive");
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->cache_seqlens || !a->workspace || !a->out ||
      !a->lse)
    return fail(MLA_ERROR_INVALID_VALUE, "a required pointer is NULL");
  if (!a->sched != !a->split_offsets)
    return fail(MLA_ERROR_INVALID_VALUE, "sched and split_offsets must both be given or both be NULL");
  if (!aligned(a->q, 16) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) || !aligned(a->out, 16) ||
      !aligned(a->workspace, 16))
    return fail(MLA_ERROR_INVALID_VALUE, "q, k_cache, v_cache, out and workspace must be 16-byte aligned");
  if (!aligned(a->lse, 4) || !aligned(a->block_table, 4) || !aligned(a->cache_seqlens, 4) ||
      !aligned(a->sched, 4) || !aligned(a->split_offsets, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "lse and the int32 arrays must be 4-byte aligned");
  if (a->kv_dtype != MLA_KV_SAME && a->kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERROR_UNSUPPORTED, "kv_dtype %d is not 0 (same as dtype) or 1 (fp8 e4m3)", a->kv_dtype);
  if (a->kv_dtype == MLA_KV_FP8_E4M3) {
    if (a->dtype != MLA_DTYPE_BF16) return fail(MLA_ERROR_UNSUPPORTED, "an fp8 cache needs dtype bf16");
    for (int i = 0; i < 3; ++i)
      if (a->k_stride[i] % 16 || a->v_stride[i] % 16)
        return fail(MLA_ERROR_INVALID_VALUE, "fp8 cache strides must be multiples of 16");
    if (!aligned(a->k_scale, 4) || !aligned(a->v_scale, 4))
      return fail(MLA_ERROR_INVALID_VALUE, "k_scale and v_scale must be 4-byte aligned");
  }
  const int64_t* strides[4] = {a->q_stride, a->k_stride, a->v_stride, a->out_stride};
  const char* names[4] = {"q_stride", "k_stride", "v_stride", "out_stride"};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if (strides[t][i] <= 0 || strides[t][i] % 8)
        return fail(MLA_ERROR_INVALID_VALUE, "%s[%d]=%lld must be a positive multiple of 8", names[t], i,
                    (long long)strides[t][i]);
  const int d = a->head_dim;
  if (a->q_stride[2] < d || a->out_stride[2] < d || a->k_stride[2] < d || a->v_stride[2] < d)
    return fail(MLA_ERROR_INVALID_VALUE, "head strides must cover a head (>= head_dim)");
  if (a->k_stride[1] < (int64_t)a->h_kv * d || a->v_stride[1] < (int64_t)a->h_kv * d)
    return fail(MLA_ERROR_INVALID_VALUE, "slot strides must cover h_kv heads");
  if ((long long)a->k_stride[1] * 2 * (MLA_PAGE_SIZE - 1) + d * 2 > 2147483647LL ||
      (long long)a->v_stride[1] * 2 * (MLA_PAGE_SIZE - 1) + d * 2 > 2147483647LL)
    return fail(MLA_ERROR_INVALID_VALUE, "slot strides too large");
  if (a->bt_stride < a->max_pages_per_seq)
    return fail(MLA_ERROR_INVALID_VALUE, "bt_stride (%lld) < max_pages_per_seq (%d)", (long long)a->bt_stride,
                a->max_pages_per_seq);
  if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f))
    return fail(MLA_ERROR_INVALID_VALUE, "softmax_scale must be finite and positive");
  if (a->causal != 0 && a->causal != 1) return fail(MLA_ERROR_INVALID_VALUE, "causal must be 0 or 1");
  const size_t need = mha_workspace_bytes(a->batch, a->s_q, a->h_q, a->h_kv, d, a->num_parts);
  if (a->workspace_bytes < need)
    return fail(MLA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the %zu required",
                a->workspace_bytes, need);
  return MLA_SUCCESS;
}

mla::MhaParams make_mha_params(const mha_decode_args* a) {
  mla::MhaParams p;
  p.q = a->q;
  p.q_s0 = a->q_stride[0]; p.q_s1 = a->q_stride[1]; p.q_s2 = a->q_stride[2];
  p.k = a->k_cache;
  p.k_s0 = a->k_stride[0]; p.k_s1 = a->k_stride[1]; p.k_s2 = a->k_stride[2];
  p.v = a->v_cache;
  p.v_s0 = a->v_stride[0]; p.v_s1 = a->v_stride[1]; p.v_s2 = a->v_stride[2];
  p.block_table = a->block_table;
  p.bt_s = a->bt_stride;
  p.seqlens = a->cache_seqlens;
  p.sched = a->sched;
  p.split_offsets = a->split_offsets;
  p.sched_f = MLA_FIXED_OVERHEAD;
  p.batch = a->batch; p.s_q = a->s_q; p.h_q = a->h_q; p.h_kv = a->h_kv;
  p.group = a->h_q / a->h_kv;
  p.rows = a->s_q * p.group;
  p.num_parts = a->num_parts;
  p.causal = a->causal;
  p.scale_log2 = a->softmax_scale * mla::kLog2e;
  p.out = a->out;
  p.o_s0 = a->out_stride[0]; p.o_s1 = a->out_stride[1]; p.o_s2 = a->out_stride[2];
  p.lse = a->lse;
  const size_t slots = (size_t)a->batch * a->h_kv + (size_t)a->num_parts;
  p.part_o = static_cast<float*>(a->workspace);
  p.part_lse = p.part_o + slots * (size_t)p.rows * a->head_dim;
  p.kv_fp8 = a->kv_dtype == MLA_KV_FP8_E4M3;
  p.k_scale = p.kv_fp8 ? a->k_scale : nullptr;
  p.v_scale = p.kv_fp8 ? a->v_scale : nullptr;
  return p;
}

}  // namespace

extern "C" {

mla_status mha_get_metadata_shape(int num_cus, int batch, int s_q, int h_q, int h_kv, int* num_parts,
                                  int* sched_elems, int* split_offsets_elems) {
  mla_status st = check_mha_shape(batch, s_q, h_q, h_kv);
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
  const int rows = s_q * (h_q / h_kv);
  const int m_blocks = (rows + kRowBlock - 1) / kRowBlock;
  int parts = num_cus / m_blocks;
  if (parts < 1) parts = 1;
  *num_parts = parts;
  *sched_elems = parts * MLA_SCHED_FIELDS;
  *split_offsets_elems = batch * h_kv + 1;
  return ok();
}

mla_status mha_get_metadata(const int32_t* cache_seqlens, int batch, int h_kv, int num_parts, int32_t* sched,
                            int32_t* split_offsets, hipStream_t stream) {
  if (batch <= 0 || h_kv <= 0) return fail(MLA_ERROR_INVALID_VALUE, "batch and h_kv must be positive");
  if ((long long)batch * h_kv > 2147483647LL / 8) return fail(MLA_ERROR_INVALID_VALUE, "batch*h_kv too large");
  if (num_parts <= 0) return fail(MLA_ERROR_INVALID_VALUE, "num_parts must be positive");
  if (!cache_seqlens || !sched || !split_offsets) return fail(MLA_ERROR_INVALID_VALUE, "NULL pointer");
  if (!aligned(cache_seqlens, 4) || !aligned(sched, 4) || !aligned(split_offsets, 4))
    return fail(MLA_ERROR_INVALID_VALUE, "int32 arrays must be 4-byte aligned");
  hipError_t e = mla::launch_metadata(cache_seqlens, batch * h_kv, h_kv, num_parts, MLA_FIXED_OVERHEAD, sched,
                                      split_offsets, stream);
  if (e != hipSuccess) return hip_fail(e, "metadata launch");
  return ok();
}

mla_status mha_workspace_size(int batch, int s_q, int h_q, int h_kv, int head_dim, int num_parts, size_t* bytes) {
  if (!bytes) return fail(MLA_ERROR_INVALID_VALUE, "bytes is NULL");
  mla_status st = check_mha_shape(batch, s_q, h_q, h_kv);
  if (st != MLA_SUCCESS) return st;
  if (head_dim <= 0 || num_parts <= 0) return fail(MLA_ERROR_INVALID_VALUE, "head_dim and num_parts must be positive");
  *bytes = mha_workspace_bytes(batch, s_q, h_q, h_kv, head_dim, num_parts);
  return ok();
}

mla_status mha_decode_splitkv(const mha_decode_args* args, hipStream_t stream) {
  mla_status st = check_mha(args);
  if (st == MLA_SUCCESS && mla::debug_checks_enabled())
    st = mla::check_paged_inputs(args->block_table, args->bt_stride, args->cache_seqlens, args->batch,
                                 args->max_pages_per_seq, args->num_pages, stream);
  if (st != MLA_SUCCESS) return st;
  hipError_t e = mla::launch_mha_splitkv(make_mha_params(args), args->dtype, args->head_dim,
                                         stream);
  if (e != hipSuccess) return hip_fail(e, "MHA split-KV launch");
  return ok();
}

mla_status mha_decode_combine(const mha_decode_args* args, hipStream_t stream) {
  mla_status st = check_mha(args);
  if (st != MLA_SUCCESS) return st;
  hipError_t e = mla::launch_mha_combine(make_mha_params(args), args->dtype, args->head_dim,
                                         stream);
  if (e != hipSuccess) return hip_fail(e, "MHA combine launch");
  return ok();
}

mla_status mha_decode(const mha_decode_args* args, hipStream_t stream) {
  mla_status st = mha_decode_splitkv(args, stream);
  if (st != MLA_SUCCESS) return st;
  return mha_decode_combine(args, stream);
}

}  // extern "C"
