// The split-KV tile scheduler's rule evaluated inside a kernel, by one wave,
// for calls that pass no precomputed schedule (page "FlashMLA: 高性能GPU注意力机制计算库
// 文件结构分析", section "6. SM资源调度优化": a per-partition quota of
// ceil(total / num_parts) plus the fixed overhead F of a piece).
//
// The rule is the one metadata_kernel applies: a nonempty unit u (a request)
// costs c_u = pages_u + F, the costs lie end to end in unit order with unit u
// starting at C_u, F0 = floor(F / 2) of its overhead positions ahead of its
// pages and F - F0 after them, and with T = sum c_u and W = ceil(T / num_parts)
// partition k owns the page positions in [kW, (k+1)W).  (A piece cut off at
// either end of a partition then misses at most half of its F on the line, so
// a cut request is split evenly.)
//
// The code below keeps the coordinates of the line with all F positions ahead
// of a unit's pages (page p of unit u at C_u + F + p); there a page lies F - F0
// further right, so partition k owns [kW + F - F0, (k+1)W + F - F0).
// Every wave that needs a partition's row, or a unit's piece slots, derives it
// from the lengths alone, so the kernels can run without the separate metadata
// launch; the results are the integers metadata_kernel writes.
//
// Because C is nondecreasing in u, "the last unit with C_u <= x" is the count
// of units with C_u <= x, less one: ballots and population counts, no search.
#pragma once

#include "mla_common.hpp"

namespace mla {

__device__ __forceinline__ int sched_cost(int n, int F) {
  const int pages = (n + kPage - 1) / kPage;
  return pages > 0 ? pages + F : 0;
}

// floor(a / w) for 0 <= a < 2^31 and w >= 1, with rw = 1 / w in double: the
// product is within one unit of the quotient, and one step corrects it.
__device__ __forceinline__ int div_floor(int a, int w, double rw) {
  int q = (int)((double)a * rw);
  q -= (long long)q * w > a;
  q += (long long)(q + 1) * w <= a;
  return q;
}

// Partitions that the pages of a unit starting at `start` with cost `cost`
// touch (0 for an empty unit); its pages lie at start + F0 + p.
__device__ __forceinline__ int sched_pieces(int start, int cost, int F, int width, double rw) {
  const int pages = cost > 0 ? cost - F : 0;
  const int first = start + (F >> 1);
  return pages > 0 ? div_floor(first + pages - 1, width, rw) - div_floor(first, width, rw) + 1 : 0;
}

// Inclusive prefix sum across the 64 lanes of a wave (all lanes active): a
// shift-and-add within each row of 16 lanes, then the row totals carried
// into the rows above by the two row broadcasts.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ int wave_total(int x) {
  return __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63);
}

__device__ __forceinline__ int count_of(uint64_t mask) { return __builtin_popcountll(mask); }

// Value of lane `last set bit of mask` (mask nonzero).
__device__ __forceinline__ int at_last(int v, uint64_t mask) {
  return __builtin_amdgcn_readlane(v, 63 - __builtin_clzll(mask));
}

// Unit lengths are read 512 at a time (eight per lane, all loads issued
// before any is used): up to 512 units, one memory round trip.
constexpr int kSchedPer = 8;
constexpr int kSchedBlock = 64 * kSchedPer;

__device__ __forceinline__ void sched_load_block(const int32_t* seqlens, int units, int rep, int u0,
                                                 int (&n)[kSchedPer]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kSchedPer; ++j) {
    const int u = u0 + j * 64 + lane;
    n[j] = u < units ? seqlens[u / rep] : 0;
  }
}

__device__ __forceinline__ int sched_total(const int32_t* seqlens, int units, int rep, int F) {
  int total = 0;
  for (int u0 = 0; u0 < units; u0 += kSchedBlock) {
    int n[kSchedPer];
    sched_load_block(seqlens, units, rep, u0, n);
    int c = 0;
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) c += sched_cost(n[j], F);
    total += wave_total(c);
  }
  return total;
}

// Partition k's row: pieces from page p0 of unit b0 to page p1 (exclusive)
// of unit b1, the first piece being piece split0 of b0; c0 = C_b0, n0 its
// length, slot0 = the piece slots of all units before b0.  b1 < b0 when the
// partition holds no page.
struct SchedRow {
  int b0, p0, b1, p1, split0, c0, n0, slot0, width;
};

__device__ __forceinline__ SchedRow sched_row(const int32_t* seqlens, int units, int rep, int parts, int F, int k) {
  const int lane = threadIdx.x & 63;
  SchedRow r = {0, 0, -1, 0, 0, 0, 0, 0, 1};
  // up to kSchedBlock units the lengths are read once and stay in registers
  const bool one = units <= kSchedBlock;
  int first[kSchedPer];
  if (one) sched_load_block(seqlens, units, rep, 0, first);
  int total;
  if (one) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) c += sched_cost(first[j], F);
    total = wave_total(c);
  } else {
    total = sched_total(seqlens, units, rep, F);
  }
  const int width = total > 0 ? (total + parts - 1) / parts : 1;
  const double rw = 1.0 / width;
  r.width = width;
  // partition k in the all-ahead coordinates (the page positions shifted by F - F0)
  const long long s = (long long)k * width + (F - (F >> 1));
  if (s >= total) return r;
  const int e = (int)min((long long)total, s + width);
  const int s32 = (int)s;
  // running over the units in order: start C of the block, piece slots of
  // the units wholly before position s, counts and last starts at or below
  // s, e - 1 and e - 1 - F
  int run = 0, slot = 0, n_s = 0, n_e = 0, n_f = 0, c_s = 0, c_e = 0, c_f = 0, len_s = 0;
  for (int u0 = 0; u0 < units; u0 += kSchedBlock) {
    int n[kSchedPer];
    if (one) {
#pragma unroll
      for (int j = 0; j < kSchedPer; ++j) n[j] = first[j];
    } else {
      sched_load_block(seqlens, units, rep, u0, n);
    }
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      if (u0 + j * 64 < units) {                  // blocks past the last unit hold nothing
        const bool in = u0 + j * 64 + lane < units;
        const int c = sched_cost(n[j], F);
        const int incl = wave_inclusive_sum(c);
        const int C = run + incl - c;
        const int pc = sched_pieces(C, c, F, width, rw);
        slot += wave_total(C + c <= s32 ? pc : 0);
        const uint64_t ms = __ballot(in && C <= s32);
        const uint64_t me = __ballot(in && C <= e - 1);
        const uint64_t mf = __ballot(in && C <= e - 1 - F);
        if (ms) { c_s = at_last(C, ms); len_s = at_last(n[j], ms); }
        if (me) c_e = at_last(C, me);
        if (mf) c_f = at_last(C, mf);
        n_s += count_of(ms);
        n_e += count_of(me);
        n_f += count_of(mf);
        run += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }
  if (c_s + F >= e) return r;                 // only the overhead of a piece falls here
  r.b0 = n_s - 1;
  r.c0 = c_s;
  r.n0 = len_s;
  r.p0 = s32 < c_s + F ? 0 : s32 - c_s - F;
  int last = e - 1, b1 = n_e - 1, cb1 = c_e;
  if (last < cb1 + F) {                       // ends inside b1's overhead: the previous unit's end
    last = cb1 - 1;
    b1 = n_f - 1;
    cb1 = c_f;
  }
  r.b1 = b1;
  r.p1 = last - cb1 - F + 1;
  r.split0 = k - (c_s + (F >> 1)) / width;  // partitions ahead of b0's first page
  r.slot0 = slot;
  return r;
}

// Piece slots, for the units u = u0 + lane of one wave: `before` = the pieces
// of all units ahead of u (split_offsets[u]), `own` = u's pieces (0 for
// u >= units, so lane units - u0 reads the total count of pieces).
__device__ __forceinline__ void sched_slots(const int32_t* seqlens, int units, int rep, int parts, int F, int u0,
                                            int& before, int& own) {
  const int lane = threadIdx.x & 63;
  if (units <= kSchedBlock) {
    // one load round: all lengths in registers, unit j * 64 + lane in n[j]
    int n[kSchedPer];
    sched_load_block(seqlens, units, rep, 0, n);
    int c[kSchedPer], t = 0;
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      c[j] = sched_cost(n[j], F);
      t += c[j];
    }
    const int total = wave_total(t);
    const int width = total > 0 ? (total + parts - 1) / parts : 1;
    const double rw = 1.0 / width;
    int run = 0, slot = 0, got_before = 0, got_own = 0;
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      if (j * 64 < units) {                       // blocks past the last unit hold nothing
        const int incl = wave_inclusive_sum(c[j]);
        const int pc = sched_pieces(run + incl - c[j], c[j], F, width, rw);
        const int pincl = wave_inclusive_sum(pc);
        // the window's lanes: unit u0 + lane sits in block j at lane (u0 + lane) - 64 j
        const int src = u0 + lane - 64 * j;
        const int bj = __builtin_amdgcn_ds_bpermute(max(0, min(63, src)) << 2, slot + pincl - pc);
        const int oj = __builtin_amdgcn_ds_bpermute(max(0, min(63, src)) << 2, pc);
        if (src >= 0 && src < 64) {
          got_before = bj;
          got_own = oj;
        }
        slot += __builtin_amdgcn_readlane(pincl, 63);
        run += __builtin_amdgcn_readlane(incl, 63);
      }
    }
    // units >= `units` (the lane of index `units` included) have no pieces
    // and sit after every piece: before = the total count
    const bool past = u0 + lane >= units;
    before = past ? slot : got_before;
    own = past ? 0 : got_own;
    return;
  }
  const int total = sched_total(seqlens, units, rep, F);
  const int width = total > 0 ? (total + parts - 1) / parts : 1;
  const double rw = 1.0 / width;
  const int head = min(u0, units);              // units wholly ahead of the window
  int run = 0, slot = 0;
  for (int v0 = 0; v0 < head; v0 += kSchedBlock) {
    int n[kSchedPer];
    sched_load_block(seqlens, head, rep, v0, n);
#pragma unroll
    for (int j = 0; j < kSchedPer; ++j) {
      const int c = sched_cost(n[j], F);
      const int incl = wave_inclusive_sum(c);
      slot += wave_total(sched_pieces(run + incl - c, c, F, width, rw));
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  const int u = u0 + lane;
  const int c = u < units ? sched_cost(seqlens[u / rep], F) : 0;
  const int incl = wave_inclusive_sum(c);
  own = sched_pieces(run + incl - c, c, F, width, rw);
  before = slot + wave_inclusive_sum(own) - own;
}

// The row of one partition, for a kernel that takes the schedule either
// precomputed (a row of `sched`) or derived in place (sched == nullptr): its
// units run from `begin` (from page begin_page, first piece begin_split) to
// `end` (up to page end_page).  Derived in place, it also carries the walk's
// starting state: C and the first slot of unit `begin`, that unit's length,
// and the width (see unit_slots).
struct PartRow {
  int begin, begin_page, end, end_page, begin_split, inl, start, slot, len0, width;
};

__device__ __forceinline__ PartRow part_row(const int32_t* sched, const int32_t* seqlens, int units, int rep,
                                            int parts, int F, int k) {
  PartRow w;
  w.inl = sched == nullptr;
  if (w.inl) {
    const SchedRow r = sched_row(seqlens, units, rep, parts, F, k);
    w.begin = r.b0; w.begin_page = r.p0; w.end = r.b1; w.end_page = r.p1; w.begin_split = r.split0;
    w.start = r.c0; w.slot = r.slot0; w.len0 = r.n0; w.width = r.width;
  } else {
    const int32_t* sc = sched + k * 8;
    w.begin = ldu(sc + 0); w.begin_page = ldu(sc + 1);
    w.end = ldu(sc + 2); w.end_page = ldu(sc + 3); w.begin_split = ldu(sc + 4);
    w.start = w.slot = w.len0 = 0;
    w.width = 1;
  }
  return w;
}

// First piece slot and piece count of unit u with length n.  Derived in
// place, the units must be visited in order from the row's first one (also
// those the partition holds no page of), carrying `start` (C of the unit) and
// `slot` (its first slot) from one to the next; the kernel keeps both in
// plain scalars: a member read selected against a load would give the walk's
// state an address and put it in scratch memory.
__device__ __forceinline__ void unit_slots(int inl, const int32_t* split_offsets, int u, int n, int F, int width,
                                           int& start, int& slot, int& slot0, int& nsplit) {
  if (inl) {
    const int cost = sched_cost(n, F);
    const int ns = sched_pieces(start, cost, F, width, 1.0 / width);
    slot0 = slot;
    nsplit = ns;
    start += cost;
    slot += ns;
  } else {
    const int s0 = ldu(split_offsets + u);
    slot0 = s0;
    nsplit = ldu(split_offsets + u + 1) - s0;
  }
}

}  // namespace mla
