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
#include "mla_sched.hpp"
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

// Walk the pieces a scheduler partition owns, calling f(chunk) for each.  The
// partition's row comes from the precomputed schedule, or, when the call
// passed none, from the scheduler's rule evaluated by this wave on the
// request lengths.
template <typename F>
__device__ __forceinline__ void for_each_chunk(const DecodeParams& p, F&& f) {
  const PartRow r = part_row(p.sched, p.seqlens, p.batch, 1, p.num_parts, p.sched_f, blockIdx.x);
  const int len0 = r.len0;
  int start = r.start, slot = r.slot;
  for (int b = r.begin; b <= r.end; ++b) {
    Chunk c;
    c.b = b;
    c.n = (r.inl && b == r.begin) ? len0 : ldu(p.seqlens + b);
    const int npages = (c.n + kPage - 1) / kPage;
    unit_slots(r.inl, p.split_offsets, b, c.n, p.sched_f, r.width, start, slot, c.slot0, c.nsplit);
    c.lo = (b == r.begin) ? r.begin_page : 0;
    c.hi = (b == r.end) ? r.end_page : npages;
    if (c.lo >= c.hi) continue;
    c.split = (b == r.begin) ? r.begin_split : 0;
    // the piece that starts a request records its slots for the combine
    if (r.inl && c.split == 0 && threadIdx.x == 0 && blockIdx.y == 0)
      *(u32x2*)(p.req_slots + 2 * b) = u32x2{(uint32_t)c.slot0, (uint32_t)c.nsplit};
    f(c);
  }
}

// Descriptor of physical page `phys` of the cache covering its first `valid`
// rows (none when valid <= 0).  Loads address rows through the per-lane
// offset, which the range check covers, so slots past a request's length are
// never read: they arrive as zeros (0 * NaN can then never reach P.V).
__device__ __forceinline__ BufRsrc page_of(const DecodeParams& p, int phys, int valid) {
  const int row_bytes = (int)(p.k_s1 * 2);
  return page_rsrc((const char*)p.k + (int64_t)phys * p.k_s0 * 2, valid > 0 ? (valid - 1) * row_bytes + kDK * 2 : 0);
}

// Rows of page `pg` of a request with n cached tokens that hold tokens.
__device__ __forceinline__ int page_valid_rows(int n, int pg) { return min(kPage, n - pg * kPage); }

// --------------------------------------------------------- fused merge --
// The combine folded into the split-KV kernel (the MI355X answer to launching
// the combine kernel early, page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析",
// section "辅助优化：可编程依赖启动与瓦片调度"): after a workgroup has written its
// piece of a split request, it counts itself in with a device-scope atomic, and
// the workgroup that writes the last piece of a row tile merges all of that
// tile's pieces by their LSE, LSE = log sum_k exp(LSE_k) and
// O = sum_k exp(LSE_k - LSE) O_k, then resets the counter for the next call.
// Used for requests cut into at most kFusedMaxPieces pieces: the merging
// workgroup reads every piece of its tile, which only pays while they are few.
// LDS of the merge: weights of the pieces per tile row, and the "last" flag.
template <int kRowsTile>
struct MergeLds {
  float w[kFusedMaxPieces][kRowsTile];
  int last;
};

// Called by every thread of the workgroup (it holds barriers) after the
// workgroup's piece (c.split of request c.b, tile rows row0 ..) was stored.
template <typename T, int kRowsTile, int kNThreads>
__device__ __forceinline__ void fused_merge(const DecodeParams& p, const Chunk& c, int row0,
                                            MergeLds<kRowsTile>& m) {
  const int tid = threadIdx.x;
  // Every wave waits for its own piece stores; then one thread makes them
  // visible device-wide (one release: a fence per thread would write back and
  // invalidate the cache once per wave) and counts the workgroup in.  The
  // workgroup that arrives last acquires the other pieces' stores.
  __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
  __syncthreads();
  int* ctr = p.counters + (int64_t)blockIdx.y * p.batch + c.b;
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(ctr, 1) == c.nsplit - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    m.last = last;
  }
  __syncthreads();
  if (!m.last) return;                              // uniform over the workgroup
  const int ns = c.nsplit;
  const int64_t s0 = c.slot0;
  if (tid < kRowsTile) {
    const int row = row0 + tid;
    float lk[kFusedMaxPieces];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFusedMaxPieces; ++k) {
      lk[k] = (k < ns && row < p.rows) ? p.part_lse[(s0 + k) * p.rows + row] : -INFINITY;
      mx = fmaxf(mx, lk[k]);
    }
    float e[kFusedMaxPieces], sum = 0.f;
#pragma unroll
    for (int k = 0; k < kFusedMaxPieces; ++k) {
      e[k] = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lk[k] - mx) * kLog2e);
      sum += e[k];
    }
    const float inv = mx == -INFINITY ? 0.f : 1.f / sum;
#pragma unroll
    for (int k = 0; k < kFusedMaxPieces; ++k) m.w[k][tid] = e[k] * inv;   // exp(LSE_k - LSE)
    if (row < p.rows) p.lse[(int64_t)c.b * p.rows + row] = mx == -INFINITY ? -INFINITY : mx + __logf(sum);
  }
  __syncthreads();
  // (row, 4-column) items, eight per batch and thread; every piece's loads of a
  // batch are in flight together (absent pieces reread the last one, weight 0)
  constexpr int kItems = kRowsTile * (kDV / 4) / kNThreads;
  static_assert(kItems % 8 == 0, "items per thread come in batches of eight");
#pragma unroll 1
  for (int ib = 0; ib < kItems; ib += 8) {
    f32x4 v[kFusedMaxPieces][8];
#pragma unroll
    for (int k = 0; k < kFusedMaxPieces; ++k) {
      const int64_t slot = s0 + min(k, ns - 1);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int it = tid + (ib + u) * kNThreads;
        const int row = min(row0 + (it >> 7), p.rows - 1);
        v[k][u] = *(const f32x4*)(p.part_o + (slot * p.rows + row) * kDV + (it & 127) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int it = tid + (ib + u) * kNThreads;
      const int rl = it >> 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kFusedMaxPieces; ++k) acc += m.w[k][rl] * v[k][u];
      if (row0 + rl < p.rows) store_out4<T>(p, c.b, row0 + rl, (it & 127) * 4, acc);
    }
  }
  if (tid == 0) *ctr = 0;                           // every piece has arrived: ready for the next call
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
