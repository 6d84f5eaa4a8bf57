/*
 * mla_decode.h - C ABI of the paged MLA decode library (libmla_decode.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Multi-head latent attention at decode time: for every
 * request b, new query token i < s_q and query head h < h_q,
 *     s_j  = softmax_scale * <q[b,i,h,0:576], K_j>      over visible keys j
 *     O    = sum_j softmax(s)_j * V_j,   V_j = K_j[0:512]
 *     LSE  = log sum_j exp(s_j)          (natural log)
 * where K_j is cached token j of request b, a 576-wide row (512 latent + 64
 * rope columns) stored in 64-token pages reached through a block table, and one
 * cached row serves all h_q heads.
 *   Sources: page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析"
 *   (blog.hotdry.top), sections "计算边界特性与优化方向抉择" (FLOPs
 *   2*h_q*s_q*s_k*(d_k+d_v) over 2*s_k*d_k bytes: one shared latent row per
 *   token) and "辅助优化：可编程依赖启动与瓦片调度" (a split-KV kernel, a combine
 *   kernel, a tile scheduler); page "FlashMLA: 高性能GPU注意力机制计算库
 *   文件结构分析" (hanhandi.cn), sections "项目主要功能" (bf16/fp16, paged KV
 *   cache with block size 64), "6. SM资源调度优化" (scheduler quota) and
 *   "火辣点评：FlashMLA的类设计" (only d_k = 576 / d_v = 512; errors printed
 *   followed by exit(1), which this library replaces with status codes);
 *   page "FlashAttention终极指南：如何通过动态计算图实现3倍推理加速"
 *   (cnnetsun.cn), sections "核心代码实现解析" (cache_seqlens, causal) and
 *   "问题二：精度偏差处理" (softmax LSE returned next to the output).
 *
 * Readings where the pages are silent: causal masking with s_q > 1 is
 * bottom-right aligned (token i sees keys j <= n - s_q + i); a row that sees no
 * key gets O = 0 and LSE = -inf; cache slots past a request's length and
 * block-table entries past its last page are never read.
 *
 * Conventions for every entry point.
 *  - Pointers marked "device" are HIP device pointers; the caller owns every
 *    buffer; the library allocates no device memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Entry points only
 *    enqueue work on it and never synchronise; a successful return means the
 *    work was enqueued.
 *  - Host-side argument checks happen before anything is enqueued: on failure
 *    nothing is enqueued, a status is returned and mla_last_error() describes
 *    it.  The process is never terminated.
 *  - Preconditions NOT checked on the host (violating them is undefined
 *    behaviour): 0 <= cache_seqlens[b] <= max_pages_per_seq * 64; the entries
 *    block_table[b, 0 : ceil(cache_seqlens[b] / 64)] lie in [0, num_pages)
 *    (these two are checked on the device by mla_check_paged_inputs, and by
 *    every decode entry point when the environment variable MLA_DEBUG is set);
 *    `sched` / `split_offsets`, when given, were produced by mla_get_metadata
 *    from the same cache_seqlens with the same num_parts; cache contents are
 *    finite; the total
 *    schedule cost sum_b (ceil(cache_seqlens[b] / 64) + MLA_FIXED_OVERHEAD) is
 *    below 2^31.
 *  - Thread safety: all entry points may be called concurrently; the error
 *    text is kept per thread.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type, declared here as HIP's own headers declare it so that
 * this header needs no HIP include (the same typedef repeated is allowed). */
typedef struct ihipStream_t* hipStream_t;

#define MLA_ABI_VERSION 4

#define MLA_D_K 576             /* cached row width = query width           */
#define MLA_D_V 512             /* value width: the first 512 columns       */
#define MLA_PAGE_SIZE 64        /* tokens per KV-cache page                 */
#define MLA_SCHED_FIELDS 8      /* int32 per scheduler partition            */
#define MLA_FIXED_OVERHEAD 2    /* per-piece overhead, in pages (scheduler):  */
                                /* a piece's set-up and merge cost about two    */
                                /* pages of attention on MI355X                 */
#define MLA_FUSED_MAX_PIECES 4  /* mla_decode_fused merges requests cut into */
                                /* at most this many pieces in its first kernel */

typedef enum {
  MLA_SUCCESS = 0,
  MLA_ERROR_INVALID_VALUE = 1,      /* bad pointer, size, stride or alignment  */
  MLA_ERROR_UNSUPPORTED = 2,        /* d_k != 576, d_v != 512, page != 64,      */
                                    /* h_kv != 1, unknown dtype                 */
  MLA_ERROR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERROR_HIP = 4                 /* a HIP runtime call or launch failed      */
} mla_status;

typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP16 = 1 } mla_dtype;

/* Element type of k_cache: the dtype of q (default), or fp8 e4m3 codes (OCP
 * "e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, codes 0x7F/0xFF are NaN) times a per-page fp32 scale.
 * Pages "DeepSeek开源FlashMLA全解析：性能革命背后的技术密码" (section "1.2
 * 计算模式创新：混合精度矩阵乘法") and "云上AI推理新突破：FlashMLA赋能
 * DeepSeek-V2-Lite提速16%" (section "3. 动态精度缩放") form the Q.K^T product
 * from fp8 casts of q and k and keep the softmax and the value product in 16
 * bits; here the latent cache itself is stored in fp8, converted exactly to
 * bf16 on chip, and the page scale is applied to the scores and to the
 * probabilities, which halves the bytes a memory-bound decode reads. */
/* MLA_KV_FP8_E4M3_QK8: the same fp8 cache, and the query-key product in fp8
 * as those pages describe it: each query row (one token of one head) is
 * taken to e4m3 codes with its own power-of-two scale 2^k, the smallest with
 * max|q| * 2^-k <= 448 (k = 0 for a row of zeros; the scaling is exact and
 * the rounding to nearest e4m3, ties to even, the only one), and S = Q.K^T
 * runs on the fp8 matrix instructions from the cached codes directly.  The
 * softmax and the value product are those of MLA_KV_FP8_E4M3.  The result
 * is the attention of the dequantized q over the dequantized cache; any
 * s_q*h_q. */
typedef enum { MLA_KV_SAME = 0, MLA_KV_FP8_E4M3 = 1, MLA_KV_FP8_E4M3_QK8 = 2 } mla_kv_dtype;

/* Text of the last error raised on the calling thread ("" if none); never NULL.
 * The pointer stays valid until the next call into the library on this thread.
 * Errors are reported this way instead of being printed before exit(1), the
 * handling page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析" criticises
 * in section "火辣点评：FlashMLA的类设计". */
const char* mla_last_error(void);

/* MLA_ABI_VERSION of the loaded library. */
int mla_abi_version(void);

/*
 * Tile-scheduler shape.  The scheduler (page "FlashMLA: 高性能GPU注意力机制计算库
 * 文件结构分析", section "6. SM资源调度优化") splits the work of all requests,
 * counted in 64-token pages, over `num_parts` partitions.  Each partition is
 * processed by ceil(s_q*h_q / M) workgroups, one per M-row query tile, where
 * M = 16 when s_q*h_q <= 16 and 64 otherwise.  num_parts is chosen so that
 * num_parts * ceil(s_q*h_q / M) fills the device once.
 *   num_cus              compute units to fill; 0 = query the current device.
 *   batch, s_q, h_q      > 0.   h_kv must be 1.
 *   num_parts (out)      suggested partition count (>= 1).
 *   sched_elems (out)    int32 elements of the `sched` array: num_parts * 8.
 *   split_offsets_elems (out) int32 elements of `split_offsets`: batch + 1.
 * Errors: INVALID_VALUE (sizes <= 0, null out-pointers), UNSUPPORTED (h_kv != 1),
 * HIP (device query failed).
 */
mla_status mla_get_metadata_shape(int num_cus, int batch, int s_q, int h_q, int h_kv,
                                  int* num_parts, int* sched_elems, int* split_offsets_elems);

/*
 * Build the split-KV tile schedule on the device (one small kernel).
 * A nonempty request b costs c_b = P_b + F, P_b = ceil(cache_seqlens[b] / 64),
 * F = MLA_FIXED_OVERHEAD; empty requests cost 0.  Costs are laid end to end in
 * request order, request b starting at C_b with F0 = floor(F / 2) overhead
 * units, then its pages, then the other F - F0 units, so page p of request b
 * sits at position C_b + F0 + p.  With T = sum of costs and
 * W = ceil(T / num_parts), partition k takes the pages whose positions fall in
 * [k*W, (k+1)*W).  Each partition then costs at most W + F, the page's quota
 * ceil(total / num_parts) + fixed overhead, counting F for every piece.
 *   cache_seqlens  device int32 [batch], each >= 0, with
 *                  sum_b (P_b + F) < 2^31.
 *   num_parts      >= 1 (normally from mla_get_metadata_shape).
 *   sched          device int32 [num_parts][8], written.  Row p =
 *                  (begin_req, begin_page, end_req, end_page, begin_split,
 *                   0, 0, 0): partition p covers request begin_req from page
 *                  begin_page, all requests strictly between, and request
 *                  end_req up to page end_page (exclusive); begin_split is the
 *                  index of its first piece among the pieces of begin_req.
 *                  Empty partition: (0, 0, -1, 0, 0, 0, 0, 0).
 *   split_offsets  device int32 [batch + 1], written: exclusive prefix sum of
 *                  the number of pieces of each request (0 for empty requests).
 * The result depends only on (cache_seqlens, num_parts) and is reused by every
 * layer of a decode step.  Errors: INVALID_VALUE, UNSUPPORTED, HIP.
 */
mla_status mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                            int num_parts, int32_t* sched, int32_t* split_offsets, hipStream_t stream);

/*
 * mla_get_metadata with the per-piece overhead F given explicitly, 0 <= F <= 64
 * (INVALID_VALUE otherwise), for the same quota rule of page "FlashMLA:
 * 高性能GPU注意力机制计算库 文件结构分析", section "6. SM资源调度优化".  Every F
 * gives a valid schedule for every decode entry point; F only moves the cuts
 * (mla_get_metadata uses MLA_FIXED_OVERHEAD).  The cost bound becomes
 * sum_b (P_b + F) < 2^31.
 */
mla_status mla_get_metadata_ex(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                               int num_parts, int fixed_overhead, int32_t* sched, int32_t* split_offsets,
                               hipStream_t stream);

/*
 * Bytes of device workspace the decode entry points need.  The pieces a split
 * request is cut into are merged by their LSE in a second kernel (page
 * "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析", section
 * "辅助优化：可编程依赖启动与瓦片调度": split-KV work, then a combine kernel),
 * so each piece's fp32 output and LSE are parked here.  Layout: first the arrival
 * counters of mla_decode_fused (m_blocks * batch int32, rounded up to 256 bytes;
 * m_blocks = ceil(s_q*h_q / 64), or 1 when s_q*h_q <= 16), then each
 * request's first piece slot and piece count (batch * 2 int32, rounded up to
 * 256 bytes; written by the split-KV kernel for the combine when the call
 * passes no schedule), then fp32 partial outputs and LSEs for up to
 * (batch + num_parts) request pieces of s_q*h_q rows each
 * ((batch + num_parts) * s_q * h_q * (512 + 1) * 4 bytes, rounded up to 256).
 * Errors: INVALID_VALUE.
 */
mla_status mla_workspace_size(int batch, int s_q, int h_q, int num_parts, size_t* bytes);

/* Arguments of mla_decode.  Strides are in ELEMENTS; the innermost (feature)
 * dimension of q, k_cache and out must be contiguous (stride 1). */
typedef struct {
  int dtype;                   /* mla_dtype of q, k_cache and out            */
  int batch, s_q, h_q, h_kv;   /* h_kv must be 1                              */
  int d_k, d_v, page_size;     /* must be 576, 512, 64                        */
  int num_pages;               /* pages in k_cache                            */
  int max_pages_per_seq;       /* columns of block_table                      */
  const void* q;               /* device [batch, s_q, h_q, 576]               */
  int64_t q_stride[3];         /*   strides of batch, token, head             */
  const void* k_cache;         /* device [num_pages, 64, h_kv, 576]           */
  int64_t k_stride[3];         /*   strides of page, slot, kv-head            */
  const int32_t* block_table;  /* device [batch, max_pages_per_seq]           */
  int64_t bt_stride;           /*   stride between rows                       */
  const int32_t* cache_seqlens;/* device [batch]                              */
  const int32_t* sched;        /* device, from mla_get_metadata, or NULL      */
  const int32_t* split_offsets;/* device, from mla_get_metadata, or NULL      */
  int num_parts;               /* the num_parts the schedule was built with   */
                               /* (both NULL: the kernels derive the schedule
                                  of mla_get_metadata, with MLA_FIXED_OVERHEAD
                                  and this num_parts, from cache_seqlens in
                                  place; no metadata launch, same results)  */
  float softmax_scale;         /* finite, > 0 (typically 1/sqrt(576))         */
  int causal;                  /* 0/1; bottom-right aligned when s_q > 1      */
  void* workspace;             /* device, >= mla_workspace_size bytes, 256-B aligned */
  size_t workspace_bytes;
  void* out;                   /* device [batch, s_q, h_q, 512], dtype        */
  int64_t out_stride[3];       /*   strides of batch, token, head             */
  float* lse;                  /* device [batch, s_q, h_q] fp32, contiguous   */
  int kv_dtype;                /* mla_kv_dtype of k_cache (k_stride counts its elements) */
  const float* k_scale;        /* MLA_KV_FP8_E4M3: device [num_pages] fp32, finite
                                  (K = code value * k_scale[page]); NULL means 1 */
} mla_decode_args;

/*
 * Paged MLA decode: mla_decode_splitkv followed by mla_decode_combine on
 * `stream`.  Writes out and lse for every (b, i, h), the attention defined at
 * the top of this header (page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析",
 * sections "跷跷板调度的数学重构" for the online softmax and "辅助优化：可编程依赖
 * 启动与瓦片调度" for the split-KV + combine structure; page "FlashAttention终极指南：
 * 如何通过动态计算图实现3倍推理加速", section "核心代码实现解析", for the
 * q / k_cache / block_table / cache_seqlens / softmax_scale / causal arguments).
 * An fp8 cache (kv_dtype = MLA_KV_FP8_E4M3) needs dtype bf16 (UNSUPPORTED
 * otherwise), for any s_q*h_q; k_cache is then 8-byte aligned instead of 16.
 * Alignment: q, k_cache, out must be 16-byte aligned, as must every stride
 * times the element size (q_stride[*], k_stride[0..1], out_stride[*] multiples
 * of 8); lse and the int32 arrays 4-byte aligned.
 * Schedule: with sched and split_offsets NULL, every workgroup of the two
 * kernels evaluates the scheduler's rule (see mla_get_metadata) for its own
 * partition or request from cache_seqlens, so a decode step needs no
 * mla_get_metadata call; a caller that reuses one schedule across many
 * layers may still pass it precomputed.
 * Errors: INVALID_VALUE (null pointer, exactly one of sched / split_offsets
 * NULL, non-positive size, bad stride or alignment, non-finite or
 * non-positive scale), UNSUPPORTED (dims, page size, h_kv, dtype),
 * WORKSPACE_TOO_SMALL, HIP (launch failed).
 */
mla_status mla_decode(const mla_decode_args* args, hipStream_t stream);

/*
 * First phase only: the split-KV attention kernel.  Requests handled by a single
 * partition get their final out/lse written here; the pieces of split requests
 * go to the workspace as fp32 partial outputs with their LSE.
 * (Page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析", section
 * "辅助优化：可编程依赖启动与瓦片调度": the splitkv_mla kernel.)
 * Same arguments and errors as mla_decode.
 */
mla_status mla_decode_splitkv(const mla_decode_args* args, hipStream_t stream);

/*
 * Second phase only: merge the pieces of every split request by their LSE
 *   LSE = log sum_k exp(LSE_k),  O = sum_k exp(LSE_k - LSE) * O_k
 * and write out/lse; also writes O = 0, LSE = -inf for requests with no cached
 * token.  Must follow mla_decode_splitkv with the same arguments on the same
 * stream.  (Same page and section: the combine kernel.)
 * Same arguments and errors as mla_decode.
 */
mla_status mla_decode_combine(const mla_decode_args* args, hipStream_t stream);

/*
 * Paged MLA decode with the combine folded into the split-KV kernel (the
 * counterpart of starting the combine kernel early by programmatic dependent
 * launch: page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析", section
 * "辅助优化：可编程依赖启动与瓦片调度").  Same result and arguments as mla_decode.
 * A workgroup that stores a piece of a split request counts itself in on a
 * device-scope atomic counter in the workspace; the one that stores the last
 * piece of a row tile merges the tile's pieces by their LSE and writes out/lse.
 * This is done for requests cut into at most MLA_FUSED_MAX_PIECES pieces; the
 * combine kernel, launched next on `stream`, merges the others and skips these.
 * Workspace: the counter region (its first bytes, see mla_workspace_size) must
 * be zero before the first call on a workspace and again whenever batch or
 * s_q*h_q grows (e.g. allocate it zero-filled); every call that runs to
 * completion leaves it zero.  Two calls sharing one workspace must not run
 * concurrently.  mla_decode, mla_decode_splitkv and mla_decode_combine never
 * read or write the counters.
 * Errors: as mla_decode.
 */
mla_status mla_decode_fused(const mla_decode_args* args, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mla_decode
 * with its workspace taken from a static array of MLA_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every GPU it runs on until the process ends.
 * args->workspace and args->workspace_bytes are ignored; every other argument,
 * the result and the errors are those of mla_decode, and WORKSPACE_TOO_SMALL
 * is returned (nothing enqueued) when mla_workspace_size(batch, s_q, h_q,
 * num_parts) exceeds MLA_NOALLOC_SCRATCH_BYTES.  The call allocates nothing.
 * The first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress); make it outside graph capture.  All calls on one GPU
 * share its array and it keeps the last call's contents (nothing in it has to
 * start at zero): calls that overlap in time on one GPU -- on different
 * streams, or from threads that do not order them -- race and may return
 * wrong results.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status mla_decode_noalloc(const mla_decode_args* args, hipStream_t stream);

/*
 * Debug check of the paged-cache indices on the device: every length
 * cache_seqlens[b] must lie in [0, 64 * max_pages_per_seq] and every entry
 * block_table[b, j] with j < ceil(cache_seqlens[b] / 64) in [0, num_pages);
 * entries past a request's last page are not read.  block_table is device
 * int32 [batch, bt_stride >= max_pages_per_seq], cache_seqlens device int32
 * [batch].  The call runs two small kernels on `stream`, then waits for the
 * stream (so it cannot be captured into a graph) and returns
 * MLA_ERROR_INVALID_VALUE, with the first bad entry (lowest request, then
 * column; a bad length before its columns) named in mla_last_error(), or
 * MLA_SUCCESS.  The result lives in a static per-GPU word: calls serialise on
 * a process-wide lock.  When the environment variable MLA_DEBUG is set (to
 * anything but "" or "0"), mla_decode, mla_decode_splitkv, mla_decode_fused,
 * mla_decode_noalloc and mha_decode_splitkv run this check after their host
 * checks and return its error without launching.  Bad indices are reported as
 * a status, not by ending the process: the print-and-exit(1) handling is what
 * page "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析", section
 * "火辣点评：FlashMLA的类设计", criticises.
 */
mla_status mla_check_paged_inputs(const int32_t* block_table, int64_t bt_stride, const int32_t* cache_seqlens,
                                  int batch, int max_pages_per_seq, int num_pages, hipStream_t stream);

/* Arguments of mla_merge_partials.  Strides are in ELEMENTS; the innermost
 * (feature) dimension of part_out and out must be contiguous. */
typedef struct {
  int dtype;                   /* mla_dtype of part_out and out               */
  int num_shards;              /* >= 1                                        */
  int batch, s_q, h_q;
  const void* part_out;        /* device: shard r's out, [num_shards][batch, s_q, h_q, 512] */
  int64_t part_out_stride[4];  /*   strides of shard, batch, token, head      */
  const float* part_lse;       /* device: shard r's lse, [num_shards][batch, s_q, h_q] fp32 */
  int64_t part_lse_stride;     /*   stride between shards (contiguous within) */
  void* out;                   /* device [batch, s_q, h_q, 512], dtype        */
  int64_t out_stride[3];       /*   strides of batch, token, head             */
  float* lse;                  /* device [batch, s_q, h_q] fp32, contiguous   */
} mla_merge_args;

/*
 * Merge of context-parallel shards (the one-GPU part of splitting a request's
 * cached tokens over several GPUs, each running mla_decode on its own range):
 * for every (b, i, h), with shard results O_r = out_r[b,i,h,:] and L_r =
 * lse_r[b,i,h],
 *     LSE = log sum_r exp(L_r),   O = sum_r exp(L_r - LSE) * O_r
 * -- the merge the combine kernel applies to the pieces of a split request
 * (page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析", section
 * "辅助优化：可编程依赖启动与瓦片调度").  Shards with L_r = -inf contribute
 * nothing; if every shard has -inf, O = 0 and LSE = -inf.
 * Causal masking with s_q > 1 is bottom-right aligned over the whole request,
 * so a shard that holds the request's last cached tokens runs mla_decode with
 * causal = 1 and its own length, and every other shard must end at or before
 * token n - s_q + 1 (all of its keys visible to every new token) and runs with
 * causal = 0.
 * Alignment: part_out and out 16-byte aligned, their strides multiples of 8;
 * part_lse and lse 4-byte aligned.  Nothing is allocated; the call only
 * enqueues one kernel on `stream`.
 * Errors: INVALID_VALUE (null pointer, non-positive size, bad stride or
 * alignment), UNSUPPORTED (dtype), HIP (launch failed).
 */
mla_status mla_merge_partials(const mla_merge_args* args, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
