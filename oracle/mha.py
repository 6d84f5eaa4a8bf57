"""Exact paged multi-head (grouped-query) decode attention, fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (page title, then section):
  [FA-KVCACHE]   "FlashAttention终极指南：如何通过动态计算图实现3倍推理加速"
                 (cnnetsun.cn), section "核心代码实现解析": decode attention of the
                 current queries q over a key cache and a separate value cache,
                 with per-request cached lengths (cache_seqlens) and a causal
                 flag; section "问题二：精度偏差处理": the softmax LSE returned
                 beside the output.
  [HANHANDI-FEAT] "FlashMLA: 高性能GPU注意力机制计算库 文件结构分析" (hanhandi.cn),
                 section "项目主要功能": the cache is paged in 64-token blocks
                 reached through a block table.

Readings (listed in the design notes):
  * k_cache and v_cache are [num_pages, 64, h_kv, d] and [num_pages, 64, h_kv,
    d_v]; token j of request b lives in page block_table[b, j // 64], slot
    j % 64, for every KV head.
  * h_q is a multiple of h_kv; query head h reads KV head h // (h_q / h_kv)
    (consecutive query heads share a KV head; h_kv = h_q is plain multi-head
    attention, h_kv = 1 multi-query attention).
  * scores are q.k times softmax_scale, softmax in base e, LSE in natural log;
    causal is bottom-right aligned; a row that sees no key gets O = 0 and
    LSE = -inf -- the same conventions as decode.py.
"""

from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .decode import PAGE, _f64, _i64, visible_keys


def kv_head_of(h: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head h."""
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    return h // (h_q // h_kv)


def gather_head(cache: np.ndarray, block_table_row: np.ndarray, n: int, hk: int) -> np.ndarray:
    """Dense [n, width] rows of KV head hk for request tokens 0..n-1."""
    n_pages = (n + PAGE - 1) // PAGE
    if n_pages == 0:
        return np.zeros((0, cache.shape[-1]), dtype=np.float64)
    pages = block_table_row[:n_pages]
    rows = cache[pages, :, hk, :].reshape(n_pages * PAGE, cache.shape[-1])
    return rows[:n]


def _softmax_attend(Qr, K, V, counts, scale):
    """Rows Qr [R, d] over keys K [n, d] / values V [n, d_v], row r seeing the
    first counts[r] keys.  Returns (O [R, d_v], LSE [R])."""
    R, n, d_v = Qr.shape[0], K.shape[0], V.shape[1]
    O = np.zeros((R, d_v), dtype=np.float64)
    L = np.full((R,), -np.inf, dtype=np.float64)
    if n == 0 or R == 0:
        return O, L
    S = (Qr @ K.T) * scale
    mask = np.arange(n)[None, :] < counts[:, None]
    S = np.where(mask, S, -np.inf)
    live = counts > 0
    m = np.where(live, S.max(axis=1), 0.0)
    E = np.where(mask, np.exp(S - m[:, None]), 0.0)
    l = E.sum(axis=1)
    O[live] = (E @ V)[live] / l[live, None]
    L[live] = m[live] + np.log(l[live])
    return O, L


def oracle_mha_rows(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale: float,
                    causal: bool, b: int, key_lo: int = 0, key_hi: int | None = None):
    """Request b, every token and head: (O [s_q, h_q, d_v], LSE [s_q, h_q]).
    With key_lo/key_hi only keys in [key_lo, key_hi) take part (a split of the
    key range, before the merge)."""
    qf = q if isinstance(q, np.ndarray) and q.dtype == np.float64 else _f64(q)
    kf = k_cache if isinstance(k_cache, np.ndarray) and k_cache.dtype == np.float64 else _f64(k_cache)
    vf = v_cache if isinstance(v_cache, np.ndarray) and v_cache.dtype == np.float64 else _f64(v_cache)
    bt = _i64(block_table)
    sl = _i64(cache_seqlens)
    _, s_q, h_q, d = qf.shape
    h_kv, d_v = kf.shape[2], vf.shape[-1]
    if kf.shape[1] != PAGE or vf.shape[1] != PAGE or kf.shape[-1] != d or vf.shape[2] != h_kv:
        raise ValueError("expected k_cache [pages,64,h_kv,d] and v_cache [pages,64,h_kv,d_v]")
    n = int(sl[b])
    lo = max(0, key_lo)
    hi = n if key_hi is None else min(n, key_hi)
    out = np.zeros((s_q, h_q, d_v), dtype=np.float64)
    lse = np.full((s_q, h_q), -np.inf, dtype=np.float64)
    for hk in range(h_kv):
        K = gather_head(kf, bt[b], n, hk)
        V = gather_head(vf, bt[b], n, hk)
        heads = [h for h in range(h_q) if kv_head_of(h, h_q, h_kv) == hk]
        for i in range(s_q):
            cnt = visible_keys(n, s_q, i, causal)
            sub = max(0, min(cnt, hi) - lo)
            Qr = qf[b, i, heads, :]
            counts = np.full((len(heads),), sub, dtype=np.int64)
            O, L = _softmax_attend(Qr, K[lo:max(lo, hi)], V[lo:max(lo, hi)], counts, float(softmax_scale))
            out[i, heads] = O
            lse[i, heads] = L
    return out, lse


def oracle_mha_decode(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale: float, causal: bool):
    """Full oracle: O [B, s_q, h_q, d_v] and LSE [B, s_q, h_q], float64.

    For request b, token i, head h, KV head g = h // (h_q / h_kv), n = cache_seqlens[b]:
      s_j = softmax_scale * <q[b,i,h], K[b,j,g]>   over the visible keys j,
      O   = sum_j softmax(s)_j V[b,j,g],   LSE = log sum_j e^{s_j}.
    """
    qf, kf, vf = _f64(q), _f64(k_cache), _f64(v_cache)
    B, s_q, h_q, _ = qf.shape
    out = np.zeros((B, s_q, h_q, vf.shape[-1]), dtype=np.float64)
    lse = np.full((B, s_q, h_q), -np.inf, dtype=np.float64)
    for b in range(B):
        out[b], lse[b] = oracle_mha_rows(qf, kf, vf, block_table, cache_seqlens, softmax_scale, causal, b)
    return out, lse


def brute_force_mha(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale: float,
                    causal: bool) -> Tuple[List, List]:
    """Pure-Python loops with math.fsum, for tiny shapes only.  Returns nested
    lists out[b][i][h][c], lse[b][i][h]."""
    qf = _f64(q)
    kf = _f64(k_cache)
    vf = _f64(v_cache)
    bt = _i64(block_table).tolist()
    sl = _i64(cache_seqlens).tolist()
    B, s_q, h_q, d = qf.shape
    h_kv, d_v = kf.shape[2], vf.shape[-1]
    group = h_q // h_kv
    out, lse = [], []
    for b in range(B):
        n = int(sl[b])
        ob, lb = [], []
        for i in range(s_q):
            cnt = visible_keys(n, s_q, i, causal)
            oi, li = [], []
            for h in range(h_q):
                g = h // group
                if cnt == 0:
                    oi.append([0.0] * d_v)
                    li.append(-math.inf)
                    continue
                keys = [kf[bt[b][j // PAGE], j % PAGE, g, :].tolist() for j in range(cnt)]
                vals = [vf[bt[b][j // PAGE], j % PAGE, g, :].tolist() for j in range(cnt)]
                qv = qf[b, i, h, :].tolist()
                s = [softmax_scale * math.fsum(qv[c] * keys[j][c] for c in range(d)) for j in range(cnt)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                den = math.fsum(w)
                oi.append([math.fsum(w[j] * vals[j][c] for j in range(cnt)) / den for c in range(d_v)])
                li.append(m + math.log(den))
            ob.append(oi)
            lb.append(li)
        out.append(ob)
        lse.append(lb)
    return out, lse


def oracle_mha_metadata(cache_seqlens, h_kv: int, num_parts: int):
    """Split-KV schedule of the MHA path: the units of work are the (request,
    KV head) pairs in request-major order (unit b * h_kv + g), each with its
    request's length; they are cut exactly as the MLA path cuts requests
    (metadata.py, same cost rule)."""
    from .metadata import oracle_metadata

    lens = [int(n) for n in np.repeat(_i64(cache_seqlens), int(h_kv)).tolist()]
    return oracle_metadata(lens, num_parts)
