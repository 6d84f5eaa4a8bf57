// Split-KV MLA decode attention: pieces shared by the two kernels (gfx950).
//
// What is computed (page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析",
// sections "跷跷板调度的数学重构" and "辅助优化：可编程依赖启动与瓦片调度"): for one
// request and one contiguous range of its 64-token pages, the softmax attention
// of a tile of query rows over those keys, with an online (running-maximum)
// softmax.  Scores and probabilities are kept in fp32 and exponentials use
// exp2 with log2(e) folded into the scale (page "FlashMLA: 高性能GPU注意力机制计算库
// 文件结构分析", section "4. Softmax数值稳定性优化").  A range that is a whole
// request writes the final output and LSE; a piece of a split request writes an
// fp32 partial output and its LSE for the combine kernel.
//
// Both kernels run one workgroup per (scheduler partition, tile of M query
// rows); pages stream HBM -> LDS while earlier pages are consumed (page
// "FlashMLA: ...文件结构分析", sections "1. shared memory的双缓冲技术" and
// "5. 向量化与异步优化解析").  Scores are formed as S^T = K . Q^T on 16x16x32 MFMA
// so that each lane ends up owning one query row; the output is accumulated
// as O^T = V^T . P^T, whose V^T operand comes from transposed LDS reads of the
// same page (V = first 512 columns of K), so P and the rescale factors stay in
// the lane of their row.  The narrow kernel (s_q*h_q <= 16) and the wide
// kernel (64-row tiles) are in mla_splitkv_narrow.hip and mla_splitkv_wide.hip.
#pragma once

#include "mla_common.hpp"
#include "mla_internal.h"

namespace mla {

template <typename T>
__device__ __forceinline__ void load_q_frag(const DecodeParams& p, int b, int row, int g,
                                            u32x4 (&qf)[18]) {
  if (row < p.rows) {
    const int tok = row / p.h_q;
    const int head = row - tok * p.h_q;
    const T* base = (const T*)p.q + b * p.q_s0 + tok * p.q_s1 + head * p.q_s2;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = *(const u32x4*)(base + (ks * 4 + g) * 8);
  } else {
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[ks] = u32x4{0, 0, 0, 0};
  }
}

// Store 4 consecutive output columns of one row (final output, dtype).
template <typename T>
__device__ __forceinline__ void store_out4(const DecodeParams& p, int b, int row, int col, f32x4 v) {
  const int tok = row / p.h_q;
  const int head = row - tok * p.h_q;
  T* dst = (T*)p.out + b * p.o_s0 + tok * p.o_s1 + head * p.o_s2 + col;
  u32x2 w = {Dt<T>::pack2(v[0], v[1]), Dt<T>::pack2(v[2], v[3])};
  *(u32x2*)dst = w;
}

__device__ __forceinline__ float lse_of(float m_log2, float l) {
  return l > 0.f ? (m_log2 + __log2f(l)) * kLn2 : -INFINITY;
}

// One contiguous page range [lo, hi) of request b, as read from the schedule.
struct Chunk {
  int b, n, lo, hi, split, slot0, nsplit;
};

// Walk the pieces a scheduler partition owns, calling f(chunk) for each.
template <typename F>
__device__ __forceinline__ void for_each_chunk(const DecodeParams& p, F&& f) {
  const int32_t* sc = p.sched + blockIdx.x * 8;
  const int begin_req = ldu(sc + 0), begin_page = ldu(sc + 1);
  const int end_req = ldu(sc + 2), end_page = ldu(sc + 3), begin_split = ldu(sc + 4);
  for (int b = begin_req; b <= end_req; ++b) {
    Chunk c;
    c.b = b;
    c.n = ldu(p.seqlens + b);
    const int npages = (c.n + kPage - 1) / kPage;
    c.lo = (b == begin_req) ? begin_page : 0;
    c.hi = (b == end_req) ? end_page : npages;
    if (c.lo >= c.hi) continue;
    c.split = (b == begin_req) ? begin_split : 0;
    c.slot0 = ldu(p.split_offsets + b);
    c.nsplit = ldu(p.split_offsets + b + 1) - c.slot0;
    f(c);
  }
}

// Descriptor of physical page `phys` of the cache.
__device__ __forceinline__ BufRsrc page_of(const DecodeParams& p, int phys, int page_bytes) {
  return page_rsrc((const char*)p.k + (int64_t)phys * p.k_s0 * 2, page_bytes);
}

// Cache policy of page loads: the narrow kernel reads every page once; in the
// wide kernel the row tiles of one request read the same pages and may meet in L2.
constexpr int kNarrowAux = 2;
constexpr int kWideAux = 0;

// Page loop driver: pages [lo, hi) alternate between two LDS buffers.  The loop
// is unrolled by two so that the buffer roles and the register stage a step
// uses are compile-time: step(parity, cur, nxt, pg) processes page pg from
// `cur` while the next page is written into `nxt`.
template <typename Step>
__device__ __forceinline__ void page_loop(int lo, int hi, MLA_LDS char* buf0, MLA_LDS char* buf1,
                                          Step&& step) {
  for (int pg = lo; pg < hi; pg += 2) {
    step(std::integral_constant<int, 0>{}, buf0, buf1, pg);
    if (pg + 1 >= hi) break;
    step(std::integral_constant<int, 1>{}, buf1, buf0, pg + 1);
  }
}

}  // namespace mla
