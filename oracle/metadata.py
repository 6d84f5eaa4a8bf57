"""Integer re-derivation of the split-KV tile schedule (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析" (hanhandi.cn), section
"6. SM资源调度优化": the work of all requests, counted in 64-token blocks, is
divided over num_sm_parts partitions with a per-partition quota of
ceil(total_num_blocks / num_sm_parts) + fixed_overhead_num_blocks, the fixed
overhead paying for the extra cost of each piece a request is cut into.
"FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析" (blog.hotdry.top), section
"辅助优化：可编程依赖启动与瓦片调度": a tile scheduler assigns requests and
blocks to SMs for load balance; split pieces are merged by a combine kernel.

The pages give the quota and the goal, not the assignment rule.  The reading
used here (listed in the design notes): every nonempty request b costs
P_b + F, P_b = ceil(n_b / 64) pages, F = fixed overhead; total T = sum of the
costs; quota Q = ceil(T / num_parts) + F.  Partitions are filled greedily in
request order: a request (or the rest of one) that fits in the remaining budget
is taken whole; otherwise the partition takes (budget - F) of its pages, if that
is positive, and closes.  Empty requests (n_b = 0) get no chunk and no split.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

PAGE = 64
FIXED_OVERHEAD = 5
SCHED_FIELDS = 8


def _pages(n: int) -> int:
    return (int(n) + PAGE - 1) // PAGE


def schedule_chunks(cache_seqlens: Sequence[int], num_parts: int,
                    fixed_overhead: int = FIXED_OVERHEAD) -> List[Tuple[int, int, int, int]]:
    """Chunks (part, request, first_page, end_page) in schedule order."""
    seq = [int(x) for x in cache_seqlens]
    if num_parts <= 0:
        raise ValueError("num_parts must be positive")
    F = int(fixed_overhead)
    P = [_pages(n) for n in seq]
    B = len(P)
    total = sum(p + F for p in P if p > 0)
    quota = -(-total // num_parts) + F
    chunks: List[Tuple[int, int, int, int]] = []
    b, p = 0, 0
    for part in range(num_parts):
        budget = quota
        while b < B:
            if P[b] == 0:
                b, p = b + 1, 0
                continue
            need = (P[b] - p) + F
            if need <= budget:
                chunks.append((part, b, p, P[b]))
                budget -= need
                b, p = b + 1, 0
            else:
                take = budget - F
                if take > 0:
                    chunks.append((part, b, p, p + take))
                    p += take
                break
    # every page of every request is covered (quota argument; checked here)
    if b != B:
        raise AssertionError("schedule left work unassigned")
    return chunks


def oracle_metadata(cache_seqlens: Sequence[int], num_parts: int,
                    fixed_overhead: int = FIXED_OVERHEAD):
    """Return (sched [num_parts, 8] int32, split_offsets [B+1] int32).

    sched[part] = (begin_req, begin_page, end_req, end_page, begin_split,
                   n_chunks, 0, 0)
      The part covers request begin_req from page begin_page, every request
      strictly between, and request end_req up to page end_page (exclusive);
      when begin_req == end_req the range is [begin_page, end_page).
      begin_split is the index of the part's first chunk among the chunks of
      begin_req; later requests of the part start at their split 0.
      An empty part is (0, 0, -1, 0, 0, 0, 0, 0).
    split_offsets = exclusive prefix sum of n_splits (chunks per request);
      requests with no cached token have 0 splits.
    """
    seq = [int(x) for x in cache_seqlens]
    B = len(seq)
    chunks = schedule_chunks(seq, num_parts, fixed_overhead)
    n_splits = [0] * B
    split_of_chunk = []
    for (_, b, _, _) in chunks:
        split_of_chunk.append(n_splits[b])
        n_splits[b] += 1
    sched = np.zeros((num_parts, SCHED_FIELDS), dtype=np.int32)
    sched[:, 2] = -1
    by_part = {}
    for idx, (part, b, lo, hi) in enumerate(chunks):
        by_part.setdefault(part, []).append((idx, b, lo, hi))
    for part, lst in by_part.items():
        i0, b0, lo0, _ = lst[0]
        _, b1, _, hi1 = lst[-1]
        sched[part] = (b0, lo0, b1, hi1, split_of_chunk[i0], len(lst), 0, 0)
    offsets = np.zeros((B + 1,), dtype=np.int32)
    offsets[1:] = np.cumsum(np.asarray(n_splits, dtype=np.int64)).astype(np.int32)
    return sched, offsets
