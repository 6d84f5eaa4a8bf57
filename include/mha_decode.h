/*
 * mha_decode.h - C ABI of the paged multi-head / grouped-query decode path of
 * libmla_decode.so (AMD Instinct MI355X, gfx950).  Status codes, error text
 * (mla_last_error) and the stream, ownership and thread-safety conventions are
 * those of mla_decode.h.
 *
 * What it computes.  Decode attention over separate paged key and value
 * caches: for every request b, new query token i < s_q and query head h < h_q,
 * with KV head g = h / (h_q / h_kv) and n = cache_seqlens[b],
 *     s_j  = softmax_scale * <q[b,i,h,:], K[b,j,g,:]>     over visible keys j
 *     O    = sum_j softmax(s)_j * V[b,j,g,:]
 *     LSE  = log sum_j exp(s_j)          (natural log)
 * where token j of request b lives in page block_table[b, j / 64], slot
 * j % 64, of both caches.
 *   Sources: page "FlashAttention终极指南：如何通过动态计算图实现3倍推理加速"
 *   (cnnetsun.cn), section "核心代码实现解析" (decode attention of q against a
 *   key cache and a value cache with cache_seqlens and a causal flag) and
 *   section "问题二：精度偏差处理" (the softmax LSE returned beside the output);
 *   page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析", section "项目主要功能"
 *   (paged cache in 64-token blocks through a block table); page "FlashMLA 在
 *   Hopper GPU 上的 MHA 内核调度优化解析", section "辅助优化：可编程依赖启动与瓦片调度"
 *   (split-KV kernel, combine kernel, tile scheduler).
 *
 * Readings where the pages are silent: consecutive query heads share a KV head
 * (h_kv = h_q is multi-head attention, h_kv = 1 multi-query attention);
 * causal masking with s_q > 1 is bottom-right aligned (token i sees keys
 * j <= n - s_q + i); a row that sees no key gets O = 0 and LSE = -inf; cache
 * slots past a request's length are read as zeros whatever they hold, and
 * block-table entries past its last page are never read.
 *
 * The units of work are (request, KV head) pairs, unit u = b * h_kv + g, each
 * with s_q * (h_q / h_kv) query rows; the scheduler cuts them exactly as
 * mla_get_metadata cuts MLA requests.
 *
 * Preconditions NOT checked on the host (undefined behaviour otherwise):
 * 0 <= cache_seqlens[b] <= max_pages_per_seq * 64; the entries
 * block_table[b, 0 : ceil(cache_seqlens[b] / 64)] lie in [0, num_pages)
 * (both checked on the device by mla_check_paged_inputs, and by
 * mha_decode_splitkv / mha_decode when MLA_DEBUG is set);
 * `sched` / `split_offsets`, when given, come from mha_get_metadata with the
 * same cache_seqlens, h_kv and num_parts; the schedule cost
 * h_kv * sum_b (ceil(cache_seqlens[b] / 64) + MLA_FIXED_OVERHEAD) is below 2^31.
 */
#ifndef MHA_DECODE_H
#define MHA_DECODE_H

#include "mla_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Scheduler shape.  Each partition is processed by ceil(s_q*(h_q/h_kv) / 64)
 * workgroups, one per block of up to 64 query rows of a unit; num_parts is
 * chosen so that num_parts times that fills the device once.
 *   num_cus              compute units to fill; 0 = query the current device.
 *   batch, s_q, h_q, h_kv   > 0, h_q a multiple of h_kv.
 *   num_parts (out)      suggested partition count (>= 1).
 *   sched_elems (out)    int32 elements of `sched`: num_parts * 8.
 *   split_offsets_elems (out)  int32 elements of `split_offsets`: batch*h_kv + 1.
 * Errors: INVALID_VALUE (sizes, null out-pointers, h_q not a multiple of
 * h_kv), HIP (device query failed).
 */
mla_status mha_get_metadata_shape(int num_cus, int batch, int s_q, int h_q, int h_kv, int* num_parts,
                                  int* sched_elems, int* split_offsets_elems);

/*
 * Build the split-KV schedule of the batch*h_kv units on the device (one
 * small kernel): unit u has length cache_seqlens[u / h_kv] and is cut by the
 * rule of mla_get_metadata (cost ceil(n / 64) + MLA_FIXED_OVERHEAD per nonempty unit, costs
 * laid end to end in unit order with the overhead split around each unit's
 * pages, partition k takes the positions in [k*W, (k+1)*W),
 * W = ceil(total / num_parts)).  sched rows and split_offsets
 * [batch*h_kv + 1] have the format of mla_get_metadata, with units in place of
 * requests.  Errors: INVALID_VALUE, HIP.
 */
mla_status mha_get_metadata(const int32_t* cache_seqlens, int batch, int h_kv, int num_parts, int32_t* sched,
                            int32_t* split_offsets, hipStream_t stream);

/*
 * Bytes of device workspace mha_decode needs: fp32 partial outputs and LSEs
 * for up to (batch*h_kv + num_parts) unit pieces of s_q*(h_q/h_kv) rows each,
 * (batch*h_kv + num_parts) * s_q*(h_q/h_kv) * (head_dim + 1) * 4 bytes,
 * rounded up to 256.  Errors: INVALID_VALUE.
 */
mla_status mha_workspace_size(int batch, int s_q, int h_q, int h_kv, int head_dim, int num_parts, size_t* bytes);

/* Arguments of mha_decode.  Strides are in ELEMENTS; the innermost (feature)
 * dimension of q, the caches and out must be contiguous (stride 1). */
typedef struct {
  int dtype;                   /* mla_dtype of q, both caches and out         */
  int batch, s_q, h_q, h_kv;   /* h_q a multiple of h_kv                      */
  int head_dim;                /* 64, 128 or 256; the same for K and V        */
  int page_size;               /* must be 64                                  */
  int num_pages;               /* pages in each cache                         */
  int max_pages_per_seq;       /* columns of block_table                      */
  const void* q;               /* device [batch, s_q, h_q, head_dim]          */
  int64_t q_stride[3];         /*   strides of batch, token, head             */
  const void* k_cache;         /* device [num_pages, 64, h_kv, head_dim]      */
  int64_t k_stride[3];         /*   strides of page, slot, KV head            */
  const void* v_cache;         /* device [num_pages, 64, h_kv, head_dim]      */
  int64_t v_stride[3];         /*   strides of page, slot, KV head            */
  const int32_t* block_table;  /* device [batch, max_pages_per_seq]           */
  int64_t bt_stride;           /*   stride between rows                       */
  const int32_t* cache_seqlens;/* device [batch]                              */
  const int32_t* sched;        /* device, from mha_get_metadata, or NULL      */
  const int32_t* split_offsets;/* device, from mha_get_metadata, or NULL      */
  int num_parts;               /* the num_parts the schedule was built with   */
                               /* (both NULL: the kernels derive the schedule
                                  of mha_get_metadata for this num_parts from
                                  cache_seqlens in place, as mla_decode does) */
  float softmax_scale;         /* finite, > 0 (typically 1/sqrt(head_dim))    */
  int causal;                  /* 0/1; bottom-right aligned when s_q > 1      */
  void* workspace;             /* device, >= mha_workspace_size bytes, 256-B aligned */
  size_t workspace_bytes;
  void* out;                   /* device [batch, s_q, h_q, head_dim], dtype   */
  int64_t out_stride[3];       /*   strides of batch, token, head             */
  float* lse;                  /* device [batch, s_q, h_q] fp32, contiguous   */
  /* Cache element type (mla_kv_dtype).  MLA_KV_SAME: both caches hold
   * `dtype`.  MLA_KV_FP8_E4M3: both hold fp8 e4m3 codes (one byte each,
   * strides still in elements) and the cached values are
   *     K = code * k_scale[page * h_kv + g],  V = code * v_scale[page * h_kv + g]
   * for physical page `page` and KV head g; requires dtype bf16 and every
   * cache stride a multiple of 16.  Source: page "FlashMLA: 高性能GPU注意力机制
   * 计算库 文件结构分析", section "项目主要功能" (FP8 KV cache); the scale
   * granularity of one per page and KV head is this library's choice. */
  int kv_dtype;
  const float* k_scale;        /* device [num_pages, h_kv] fp32, finite; NULL means 1 */
  const float* v_scale;        /* device [num_pages, h_kv] fp32, finite; NULL means 1 */
} mha_decode_args;

/*
 * Paged MHA/GQA decode: mha_decode_splitkv then mha_decode_combine on
 * `stream`.  Writes out and lse for every (b, i, h).
 * Alignment: q, both caches, out and workspace 16-byte aligned; every stride
 * a positive multiple of 8 elements; lse and the int32 arrays 4-byte aligned.
 * Errors: INVALID_VALUE (null pointer, exactly one of sched / split_offsets
 * NULL, non-positive size, bad stride or alignment, non-finite or
 * non-positive scale, h_q not a multiple of h_kv), UNSUPPORTED (dtype,
 * head_dim, page size), WORKSPACE_TOO_SMALL, HIP.
 */
mla_status mha_decode(const mha_decode_args* args, hipStream_t stream);
/* (also UNSUPPORTED: an fp8 cache with dtype other than bf16, or a kv_dtype
 * this library does not know; INVALID_VALUE: an fp8 cache stride not a
 * multiple of 16, a misaligned scale array) */

/* First phase only: the split-KV kernel (whole units get their final out/lse,
 * pieces of split units go to the workspace).  Same arguments and errors. */
mla_status mha_decode_splitkv(const mha_decode_args* args, hipStream_t stream);

/* Second phase only: merge of the split units' pieces by their LSE, and
 * O = 0 / LSE = -inf for requests with no cached token.  Must follow
 * mha_decode_splitkv with the same arguments on the same stream. */
mla_status mha_decode_combine(const mha_decode_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MHA_DECODE_H */
