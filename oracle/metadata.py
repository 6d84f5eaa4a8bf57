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

The pages give the quota and the goal, not the assignment rule.  Reading used
here (listed in the design notes): every nonempty request b costs c_b = P_b + F
(P_b = ceil(n_b / 64) pages, F = fixed overhead), empty requests cost 0.  The
costs are laid end to end on one line in request order, request b occupying
[C_b, C_b + c_b): F0 = floor(F / 2) overhead units, one unit per page, then the
other F - F0 overhead units, so page p of request b sits at position
C_b + F0 + p.  With T = sum of the costs and Q' = ceil(T / num_parts),
partition k takes every page whose position lies in [k Q', (k+1) Q').

Every piece pays F in the kernel, but the line holds F once per request: a
piece that begins or ends at a cut gets only part of its F from the line.
With the overhead on both sides of a request's pages, the two pieces at a cut
lack F - F0 and F0 respectively instead of 0 and F, so a request cut in two
is cut in the middle (e.g. 64 pages with F = 2: 32 + 32 rather than 31 + 33).
A partition lacks at most F0 at its first piece and F - F0 at its last, so its
cost never exceeds the quota Q' + F.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

PAGE = 64
# F, in pages.  The page names a fixed overhead but gives no value; this one
# is the library's MLA_FIXED_OVERHEAD (set from the measured cost of a piece).
FIXED_OVERHEAD = 2
SCHED_FIELDS = 8
EMPTY_PART = [0, 0, -1, 0, 0, 0, 0, 0]


def _pages(n: int) -> int:
    return (int(n) + PAGE - 1) // PAGE


def schedule_chunks(cache_seqlens: Sequence[int], num_parts: int,
                    fixed_overhead: int = FIXED_OVERHEAD) -> List[Tuple[int, int, int, int]]:
    """Pieces (part, request, first_page, end_page), ordered by part then request."""
    if num_parts <= 0:
        raise ValueError("num_parts must be positive")
    F = int(fixed_overhead)
    F0 = F // 2                     # overhead units ahead of a request's pages
    P = [_pages(n) for n in cache_seqlens]
    start = 0                       # C_b: where request b begins on the cost line
    total = sum(p + F for p in P if p > 0)
    width = max(1, -(-total // num_parts))      # Q' = ceil(T / num_parts)
    chunks: List[Tuple[int, int, int, int]] = []
    for b, p_b in enumerate(P):
        if p_b == 0:
            continue
        for page in range(p_b):
            part = (start + F0 + page) // width
            if chunks and chunks[-1][0] == part and chunks[-1][1] == b:
                chunks[-1] = (part, b, chunks[-1][2], page + 1)
            else:
                chunks.append((part, b, page, page + 1))
        start += p_b + F
    chunks.sort(key=lambda c: (c[0], c[1]))
    return chunks


def oracle_metadata(cache_seqlens: Sequence[int], num_parts: int,
                    fixed_overhead: int = FIXED_OVERHEAD):
    """Return (sched [num_parts, 8] int32, split_offsets [B+1] int32).

    sched[part] = (begin_req, begin_page, end_req, end_page, begin_split, 0, 0, 0)
      The part covers request begin_req from page begin_page, every request
      strictly between, and request end_req up to page end_page (exclusive);
      when begin_req == end_req the range is [begin_page, end_page).
      begin_split is the index of the part's first piece among the pieces of
      begin_req; later requests of the part start at their piece 0.
      An empty part is (0, 0, -1, 0, 0, 0, 0, 0).
    split_offsets = exclusive prefix sum of n_splits (pieces per request);
      requests with no cached token have 0 pieces.
    """
    B = len(cache_seqlens)
    chunks = schedule_chunks(cache_seqlens, num_parts, fixed_overhead)
    pieces = [[] for _ in range(B)]
    for ch in sorted(chunks, key=lambda c: (c[1], c[2])):
        pieces[ch[1]].append(ch)
    sched = np.tile(np.asarray(EMPTY_PART, dtype=np.int32), (num_parts, 1))
    by_part = {}
    for ch in chunks:
        by_part.setdefault(ch[0], []).append(ch)
    for part, lst in by_part.items():
        first, last = lst[0], lst[-1]
        sched[part] = (first[1], first[2], last[1], last[3], pieces[first[1]].index(first), 0, 0, 0)
    offsets = np.zeros((B + 1,), dtype=np.int32)
    offsets[1:] = np.cumsum(np.asarray([len(x) for x in pieces], dtype=np.int64)).astype(np.int32)
    return sched, offsets
