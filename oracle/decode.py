"""Exact MLA decode attention over a paged latent KV cache (fp64 CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (page title, then section):
  [HOTDRY-ROOF]    "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析" (blog.hotdry.top),
                   section "计算边界特性与优化方向抉择": the FLOP count
                   2*h_q*s_q*s_k*(d_k+d_v) against 2*s_k*d_k bytes, i.e. every
                   query head reads the same single cached latent row per token.
  [HOTDRY-SEESAW]  same page, section "跷跷板调度的数学重构": online softmax with a
                   running maximum m (initially -inf) and output o (initially 0),
                   scores p = q K^T scaled by the softmax scale; its result equals
                   the plain softmax-weighted sum, which is what is written here.
  [HANHANDI-FEAT]  "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析" (hanhandi.cn),
                   section "项目主要功能": bf16/fp16 inputs, paged KV cache with
                   64-token blocks; section "火辣点评：FlashMLA的类设计": query
                   width fixed at 576 and value width at 512.
  [FA-KVCACHE]     "FlashAttention终极指南：如何通过动态计算图实现3倍推理加速"
                   (cnnetsun.cn), sections "核心代码实现解析" (cache_seqlens,
                   causal) and "问题二：精度偏差处理" (the softmax LSE returned
                   beside the output for checking).

Readings where the pages are silent (each one is listed in the design notes):
  * V is the first 512 columns of the same cached 576-wide row (one shared
    latent KV head for all h_q query heads).
  * scores are q.k multiplied by softmax_scale; softmax in base e; LSE is the
    natural-log log-sum-exp of the scaled scores.
  * causal with s_q > 1 is bottom-right aligned: new token i (0-based) of a
    request with n cached tokens sees keys j <= n - s_q + i.
  * a row that sees no key returns O = 0 and LSE = -inf.
  * cache slots at positions >= n, and block-table entries past the last used
    page, never influence the result.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np

D_K = 576   # cached row width: 512 latent + 64 rope  [HANHANDI-FEAT]
D_V = 512   # value width: the first 512 columns of the row  [HANHANDI-FEAT]
PAGE = 64   # tokens per KV-cache page  [HANHANDI-FEAT]


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp16/fp32) or array to float64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def visible_keys(n: int, s_q: int, i: int, causal: bool) -> int:
    """Number of cached keys that new token i of a request with n cached tokens
    attends to.  Keys are always a prefix 0..count-1 of the request's tokens.
    Non-causal: all n.  Causal (bottom-right aligned): j <= n - s_q + i."""
    if not causal:
        return n
    return max(0, min(n, n - s_q + i + 1))


def gather_rows(k_cache: np.ndarray, block_table_row: np.ndarray, n: int) -> np.ndarray:
    """Dense [n, 576] float64 matrix of request tokens 0..n-1: token j lives in
    page block_table_row[j // 64], slot j % 64  [HANHANDI-FEAT]."""
    n_pages = (n + PAGE - 1) // PAGE
    if n_pages == 0:
        return np.zeros((0, k_cache.shape[-1]), dtype=np.float64)
    pages = block_table_row[:n_pages]
    rows = k_cache[pages, :, 0, :].reshape(n_pages * PAGE, k_cache.shape[-1])
    return rows[:n]


def _attend(Qr: np.ndarray, K: np.ndarray, counts: np.ndarray, scale: float):
    """Softmax attention of rows Qr [R, 576] over the prefixes K[:counts[r]].

    Returns (O [R, 512], LSE [R]) in float64.  [HOTDRY-ROOF], [HOTDRY-SEESAW]
    """
    R = Qr.shape[0]
    O = np.zeros((R, D_V), dtype=np.float64)
    L = np.full((R,), -np.inf, dtype=np.float64)
    n = K.shape[0]
    if n == 0 or R == 0:
        return O, L
    S = (Qr @ K.T) * scale                               # scaled scores [R, n]
    mask = np.arange(n)[None, :] < counts[:, None]       # visible keys per row
    S = np.where(mask, S, -np.inf)
    live = counts > 0
    m = np.where(live, S.max(axis=1), 0.0)                # row maximum
    E = np.where(mask, np.exp(S - m[:, None]), 0.0)       # exp(s - m)
    l = E.sum(axis=1)                                     # softmax denominator
    O_live = (E @ K[:, :D_V])                             # V = first 512 columns
    O[live] = O_live[live] / l[live, None]
    L[live] = m[live] + np.log(l[live])
    return O, L


def oracle_decode_rows(q, k_cache, block_table, cache_seqlens, softmax_scale: float,
                       causal: bool, b: int, rows: Sequence[int] | None = None):
    """Oracle output of request b for the query rows ``rows`` (row r is
    token r // h_q, head r % h_q; default all s_q*h_q rows).

    Returns (O [len(rows), 512], LSE [len(rows)]) float64.  Inputs may be the
    torch tensors handed to the GPU (bf16/fp16 values are upcast exactly) or
    pre-converted float64/int64 arrays.
    """
    qf = _f64(q) if not isinstance(q, np.ndarray) or q.dtype != np.float64 else q
    kf = _f64(k_cache) if not isinstance(k_cache, np.ndarray) or k_cache.dtype != np.float64 else k_cache
    bt = _i64(block_table)
    sl = _i64(cache_seqlens)
    _, s_q, h_q, d = qf.shape
    if d != D_K or kf.shape[-1] != D_K or kf.shape[1] != PAGE or kf.shape[2] != 1:
        raise ValueError("expected q [B,s_q,h_q,576] and k_cache [pages,64,1,576]")
    R = s_q * h_q
    rows = np.arange(R) if rows is None else np.asarray(list(rows), dtype=np.int64)
    n = int(sl[b])
    K = gather_rows(kf, bt[b], n)
    Qr = qf[b].reshape(R, D_K)[rows]
    counts = np.array([visible_keys(n, s_q, int(r) // h_q, causal) for r in rows], dtype=np.int64)
    return _attend(Qr, K, counts, float(softmax_scale))


def oracle_decode(q, k_cache, block_table, cache_seqlens, softmax_scale: float, causal: bool):
    """Full oracle: O [B, s_q, h_q, 512] and LSE [B, s_q, h_q], float64.

    For request b, token i, head h, with n = cache_seqlens[b]:
      K_j = cached row j (through the block table), V_j = K_j[:512],
      s_j = softmax_scale * <q[b,i,h], K_j>,
      O   = sum_j softmax(s)_j V_j over the visible keys, LSE = log sum_j e^{s_j}.
    """
    qf = _f64(q)
    kf = _f64(k_cache)
    bt = _i64(block_table)
    sl = _i64(cache_seqlens)
    B, s_q, h_q, _ = qf.shape
    out = np.zeros((B, s_q, h_q, D_V), dtype=np.float64)
    lse = np.full((B, s_q, h_q), -np.inf, dtype=np.float64)
    for b in range(B):
        O, L = oracle_decode_rows(qf, kf, bt, sl, softmax_scale, causal, b)
        out[b] = O.reshape(s_q, h_q, D_V)
        lse[b] = L.reshape(s_q, h_q)
    return out, lse


def oracle_partial(q, k_cache, block_table, cache_seqlens, softmax_scale: float,
                   causal: bool, b: int, key_lo: int, key_hi: int):
    """Attention of request b restricted to keys j in [key_lo, key_hi) (and the
    usual visibility).  Returns the normalised partial output and its LSE, the
    quantities a split of the key range produces before the merge
    (page "FlashMLA 在 Hopper GPU 上的 MHA 内核调度优化解析", section
    "辅助优化：可编程依赖启动与瓦片调度": split-KV work followed by a combine)."""
    qf = _f64(q)
    kf = _f64(k_cache)
    bt = _i64(block_table)
    sl = _i64(cache_seqlens)
    _, s_q, h_q, _ = qf.shape
    R = s_q * h_q
    n = int(sl[b])
    K = gather_rows(kf, bt[b], n)
    Qr = qf[b].reshape(R, D_K)
    lo, hi = max(0, key_lo), min(n, key_hi)
    counts = np.array([visible_keys(n, s_q, r // h_q, causal) for r in range(R)], dtype=np.int64)
    # keys of the slice that row r sees: [lo, min(hi, counts[r]))
    sub_counts = np.clip(np.minimum(counts, hi) - lo, 0, None)
    return _attend(Qr, K[lo:max(lo, hi)], sub_counts, float(softmax_scale))


def oracle_merge(parts: Iterable[Tuple[np.ndarray, np.ndarray]]):
    """Merge partial results (O_k normalised, LSE_k) of disjoint key subsets:
    LSE = log sum_k e^{LSE_k},  O = sum_k e^{LSE_k - LSE} O_k.
    Parts whose LSE is -inf carry no weight; if all are -inf, O = 0, LSE = -inf."""
    parts = list(parts)
    lses = np.stack([p[1] for p in parts], axis=0)           # [k, R]
    Os = np.stack([p[0] for p in parts], axis=0)             # [k, R, 512]
    top = lses.max(axis=0)
    live = np.isfinite(top)
    top_safe = np.where(live, top, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - top_safe[None, :]), 0.0)
    tot = w.sum(axis=0)
    L = np.where(live, top_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    O = np.zeros(Os.shape[1:], dtype=np.float64)
    O[live] = (np.einsum("kr,krc->rc", w, Os)[live]) / tot[live, None]
    return O, L


def brute_force_decode(q, k_cache, block_table, cache_seqlens, softmax_scale: float,
                       causal: bool) -> Tuple[List, List]:
    """Pure-Python triple loop with math.fsum, for tiny shapes only.

    Independent of NumPy's BLAS: every score, weight and output element is a
    correctly rounded sum.  Returns nested lists out[b][i][h][c], lse[b][i][h].
    """
    qf = _f64(q).tolist()
    kf = _f64(k_cache)
    bt = _i64(block_table).tolist()
    sl = _i64(cache_seqlens).tolist()
    B = len(qf)
    s_q = len(qf[0])
    h_q = len(qf[0][0])
    out, lse = [], []
    for b in range(B):
        n = int(sl[b])
        rows_b = []
        for j in range(n):
            page = bt[b][j // PAGE]
            rows_b.append(kf[page, j % PAGE, 0, :].tolist())
        ob, lb = [], []
        for i in range(s_q):
            oi, li = [], []
            cnt = visible_keys(n, s_q, i, causal)
            for h in range(h_q):
                qv = qf[b][i][h]
                if cnt == 0:
                    oi.append([0.0] * D_V)
                    li.append(-math.inf)
                    continue
                s = [softmax_scale * math.fsum(qv[d] * rows_b[j][d] for d in range(D_K))
                     for j in range(cnt)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                den = math.fsum(w)
                oi.append([math.fsum(w[j] * rows_b[j][c] for j in range(cnt)) / den
                           for c in range(D_V)])
                li.append(m + math.log(den))
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return out, lse
