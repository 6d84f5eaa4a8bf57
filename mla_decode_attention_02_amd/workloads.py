"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can consume what
it produces.

Layout (shared by every consumer):
  q            [B, s_q, h_q, 576]        bf16/fp16
  k_cache      [num_pages, 64, 1, 576]   bf16/fp16   (one latent KV head)
  block_table  [B, max_pages]            int32       (-1 past a request's pages)
  cache_seqlens[B]                       int32

Recipe (fixed so that every run reproduces the same tensors):
  g = torch.Generator('cpu').manual_seed(seed), then in this order
    1. seqlens: fixed list, or torch.randint(lo, hi + 1, (B,), generator=g)
    2. perm = torch.randperm(N, generator=g), N = sum_b ceil(n_b / 64) + extra
       pages; request b takes the next ceil(n_b / 64) entries of perm
    3. q = torch.randn(B, s_q, h_q, 576, generator=g) * sigma
    4. k = torch.randn(N, 64, 1, 576, generator=g) * sigma
    5. both cast to the dtype (round to nearest even)
  Optional poison (correctness runs only): cache slots at positions >= n_b in a
  request's last page, and every page no request uses, are overwritten with
  +-POISON along the sign of the request's first query row, so that any read of
  them would dominate the softmax and the output.
  fp8 cache (kv_dtype="fp8", bf16 q only): step 4's fp32 k (poisoned as above)
  is encoded per page as fp8 e4m3fn codes and one fp32 scale per page:
    amax_p = max |k[p]|, scale_p = amax_p / 448 ("amax"), or the power of two
    2^ceil(log2(amax_p / 448)) ("pow2"), or no scale tensor at all ("none",
    codes = k cast directly); codes = clamp(k / scale_p, +-448) cast with
    torch's float8_e4m3fn rounding.  The codes and scales are the inputs; the
    values they stand for are code value * scale_p.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch

D_K = 576
D_V = 512
PAGE = 64
POISON = 64.0

_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shapes, distribution, seed)."""

    name: str
    batch: int
    s_q: int
    h_q: int
    dtype: str
    sigma: float
    causal: bool
    seqlens: Optional[Sequence[int]] = None      # fixed lengths, or
    seqlen_range: Optional[tuple] = None          # inclusive (lo, hi) uniform integers
    seed: int = 0
    kv: str = "same"                              # "same" (dtype) or "fp8" (e4m3 codes + page scales)
    qk8: bool = False                             # fp8 cache and the fp8 query-key product
    description: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.s_q * self.h_q


# The workloads the measurements are quoted on.  Seeds are the index, except
# for the fp8-cache variants 6, 11 and 12: workloads 3, 2 and 5 (same seed,
# lengths and page table) with an fp8 cache, and 13, 14 and 15: workloads
# 11, 12 and 6 with the fp8 query-key product as well.  (7..10 are the MHA
# workloads.)
WORKLOADS = {
    1: Workload("tiny", 2, 1, 16, "bf16", 1.0, False, seqlens=(64, 100), seed=1,
                description="B2 s_q1 h_q16 bf16, s_k {64,100}, non-causal"),
    2: Workload("bs64_hq128_sk4096", 64, 1, 128, "bf16", 1.0, False, seqlens=(4096,) * 64, seed=2,
                description="B64 s_q1 h_q128 bf16, every s_k 4096"),
    3: Workload("varlen_bs128_hq16", 128, 1, 16, "bf16", 1.0, False, seqlen_range=(1, 8192), seed=3,
                description="B128 s_q1 h_q16 bf16, s_k ~ U[1,8192]"),
    4: Workload("multitoken_bs32_sq2_hq128", 32, 2, 128, "fp16", 0.5, True,
                seqlen_range=(12288, 16384), seed=4,
                description="B32 s_q2 h_q128 fp16 causal, s_k ~ U[12288,16384], sigma 0.5"),
    5: Workload("longctx_bs4_hq128", 4, 1, 128, "bf16", 1.0, False,
                seqlens=(65536, 98304, 131072, 131072), seed=5,
                description="B4 s_q1 h_q128 bf16, s_k {64K,96K,128K,128K}"),
    6: Workload("varlen_bs128_hq16_fp8kv", 128, 1, 16, "bf16", 1.0, False, seqlen_range=(1, 8192), seed=3,
                kv="fp8",
                description="B128 s_q1 h_q16 bf16 q, fp8 e4m3 KV with per-page scales, s_k ~ U[1,8192]"),
    11: Workload("bs64_hq128_sk4096_fp8kv", 64, 1, 128, "bf16", 1.0, False, seqlens=(4096,) * 64, seed=2,
                 kv="fp8",
                 description="B64 s_q1 h_q128 bf16 q, fp8 e4m3 KV with per-page scales, every s_k 4096"),
    12: Workload("longctx_bs4_hq128_fp8kv", 4, 1, 128, "bf16", 1.0, False,
                 seqlens=(65536, 98304, 131072, 131072), seed=5, kv="fp8",
                 description="B4 s_q1 h_q128 bf16 q, fp8 e4m3 KV with per-page scales, s_k {64K,96K,128K,128K}"),
    13: Workload("bs64_hq128_sk4096_fp8kv_qk8", 64, 1, 128, "bf16", 1.0, False, seqlens=(4096,) * 64, seed=2,
                 kv="fp8", qk8=True,
                 description="workload 11 with q taken into fp8 (per-row power-of-two scale) for an fp8 Q.K^T"),
    14: Workload("longctx_bs4_hq128_fp8kv_qk8", 4, 1, 128, "bf16", 1.0, False,
                 seqlens=(65536, 98304, 131072, 131072), seed=5, kv="fp8", qk8=True,
                 description="workload 12 with q taken into fp8 (per-row power-of-two scale) for an fp8 Q.K^T"),
    15: Workload("varlen_bs128_hq16_fp8kv_qk8", 128, 1, 16, "bf16", 1.0, False, seqlen_range=(1, 8192), seed=3,
                 kv="fp8", qk8=True,
                 description="workload 6 with q taken into fp8 (per-row power-of-two scale) for an fp8 Q.K^T"),
}


@dataclass
class DecodeInputs:
    q: torch.Tensor
    k_cache: torch.Tensor
    block_table: torch.Tensor
    cache_seqlens: torch.Tensor
    softmax_scale: float
    causal: bool
    dtype: str
    k_scale: Optional[torch.Tensor] = None       # fp8 cache: [num_pages] fp32

    def to(self, device) -> "DecodeInputs":
        return DecodeInputs(self.q.to(device), self.k_cache.to(device),
                            self.block_table.to(device), self.cache_seqlens.to(device),
                            self.softmax_scale, self.causal, self.dtype,
                            None if self.k_scale is None else self.k_scale.to(device))


def pages_of(n: int) -> int:
    return (int(n) + PAGE - 1) // PAGE


def make_inputs(batch: int, s_q: int, h_q: int, dtype: str = "bf16", *,
                seqlens: Optional[Sequence[int]] = None,
                seqlen_range: Optional[tuple] = None,
                sigma: float = 1.0, causal: bool = False, seed: int = 0,
                extra_pages: int = 0, poison: bool = False,
                max_pages: Optional[int] = None, kv_dtype: str = "same",
                scale_mode: str = "amax") -> DecodeInputs:
    """Draw one seeded workload following the recipe in the module docstring."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    if kv_dtype not in ("same", "fp8"):
        raise ValueError("kv_dtype must be 'same' or 'fp8'")
    if kv_dtype == "fp8" and dtype != "bf16":
        raise ValueError("an fp8 cache goes with a bf16 q")
    if scale_mode not in ("amax", "pow2", "none"):
        raise ValueError("scale_mode must be 'amax', 'pow2' or 'none'")
    g = torch.Generator("cpu").manual_seed(int(seed))
    if seqlens is not None:
        sl = torch.tensor([int(x) for x in seqlens], dtype=torch.int64)
        if sl.numel() != batch:
            raise ValueError("len(seqlens) != batch")
    elif seqlen_range is not None:
        lo, hi = seqlen_range
        sl = torch.randint(int(lo), int(hi) + 1, (batch,), generator=g, dtype=torch.int64)
    else:
        raise ValueError("give seqlens or seqlen_range")
    n_pages = [pages_of(n) for n in sl.tolist()]
    used = sum(n_pages)
    total = used + int(extra_pages)
    perm = torch.randperm(total, generator=g) if total > 0 else torch.zeros(0, dtype=torch.int64)
    width = max(max(n_pages) if n_pages else 0, 1)
    if max_pages is not None:
        if max_pages < width:
            raise ValueError("max_pages smaller than the longest request")
        width = max_pages
    bt = torch.full((batch, width), -1, dtype=torch.int32)
    pos = 0
    for b, p in enumerate(n_pages):
        bt[b, :p] = perm[pos:pos + p].to(torch.int32)
        pos += p
    tdt = _DTYPES[dtype]
    q = (torch.randn(batch, s_q, h_q, D_K, generator=g) * sigma).to(tdt)
    k = torch.randn(max(total, 1), PAGE, 1, D_K, generator=g) * sigma
    k_scale = None
    if kv_dtype == "fp8":
        if poison:
            _poison(q, k, bt, sl, perm[used:] if total > used else None)
        k, k_scale = _encode_fp8(k, scale_mode)
    else:
        k = k.to(tdt)
        if poison:
            _poison(q, k, bt, sl, perm[used:] if total > used else None)
    return DecodeInputs(q=q, k_cache=k, block_table=bt,
                        cache_seqlens=sl.to(torch.int32),
                        softmax_scale=1.0 / (D_K ** 0.5), causal=causal, dtype=dtype, k_scale=k_scale)


def _encode_fp8(k: torch.Tensor, scale_mode: str):
    """fp32 cache -> (e4m3fn codes, per-page fp32 scales or None)."""
    if scale_mode == "none":
        return k.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn), None
    amax = k.abs().amax(dim=(1, 2, 3)).clamp_min(1e-30)
    scale = amax / FP8_MAX
    if scale_mode == "pow2":
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    codes = (k / scale.view(-1, 1, 1, 1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale.to(torch.float32).contiguous()


def _poison(q, k, bt, sl, unused_pages):
    for b in range(q.shape[0]):
        n = int(sl[b])
        p = pages_of(n)
        direction = torch.sign(q[b, 0, 0].float())
        direction[direction == 0] = 1.0
        row = (direction * POISON).to(k.dtype)
        if p > 0 and n % PAGE != 0:
            page = int(bt[b, p - 1])
            k[page, n % PAGE:, 0, :] = row
    if unused_pages is not None and unused_pages.numel() > 0:
        k[unused_pages] = POISON


def workload_inputs(index: int, poison: bool = False, **overrides) -> DecodeInputs:
    """Inputs of one of the named workloads."""
    w = WORKLOADS[int(index)]
    kw = dict(seqlens=w.seqlens, seqlen_range=w.seqlen_range, sigma=w.sigma,
              causal=w.causal, seed=w.seed, poison=poison, kv_dtype=w.kv)
    kw.update(overrides)
    return make_inputs(w.batch, w.s_q, w.h_q, w.dtype, **kw)


# ------------------------------------------------------ general paged MHA --
@dataclass
class MhaInputs:
    """Inputs of paged multi-head / grouped-query decode attention.

      q            [B, s_q, h_q, d]             bf16/fp16
      k_cache      [num_pages, 64, h_kv, d]     bf16/fp16
      v_cache      [num_pages, 64, h_kv, d_v]   bf16/fp16
      block_table  [B, max_pages]               int32 (-1 past a request's pages)
      cache_seqlens[B]                          int32
    """
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    cache_seqlens: torch.Tensor
    softmax_scale: float
    causal: bool
    dtype: str
    k_scale: Optional[torch.Tensor] = None       # fp8 caches: [num_pages, h_kv] fp32
    v_scale: Optional[torch.Tensor] = None

    def to(self, device) -> "MhaInputs":
        mv = lambda t: None if t is None else t.to(device)
        return MhaInputs(self.q.to(device), self.k_cache.to(device), self.v_cache.to(device),
                         self.block_table.to(device), self.cache_seqlens.to(device),
                         self.softmax_scale, self.causal, self.dtype, mv(self.k_scale), mv(self.v_scale))


@dataclass(frozen=True)
class MhaWorkload:
    name: str
    batch: int
    s_q: int
    h_q: int
    h_kv: int
    head_dim: int
    dtype: str
    causal: bool
    seqlens: Optional[Sequence[int]] = None
    seqlen_range: Optional[tuple] = None
    seed: int = 0
    kv: str = "same"
    description: str = field(default="", compare=False)


# Grouped-query decode workloads (head size 128, the common LLM shape): one
# GPU's share of a 64-query-head / 8-KV-head model, and a long-context batch.
MHA_WORKLOADS = {
    7: MhaWorkload("gqa_bs64_hq64_hkv8_d128", 64, 1, 64, 8, 128, "bf16", False, seqlen_range=(1, 8192), seed=7,
                   description="B64 s_q1 h_q64 h_kv8 d128 bf16, s_k ~ U[1,8192]"),
    8: MhaWorkload("gqa_longctx_bs8_hq32_hkv8_d128", 8, 1, 32, 8, 128, "bf16", False, seqlens=(32768,) * 8,
                   seed=8, description="B8 s_q1 h_q32 h_kv8 d128 bf16, every s_k 32768"),
    9: MhaWorkload("gqa_bs64_hq64_hkv8_d128_fp8kv", 64, 1, 64, 8, 128, "bf16", False, seqlen_range=(1, 8192),
                   seed=7, kv="fp8",
                   description="workload 7 with fp8 e4m3 K/V caches, one scale per page and KV head"),
    10: MhaWorkload("mqa_bs128_hq64_hkv1_d128", 128, 1, 64, 1, 128, "bf16", False, seqlen_range=(1, 8192),
                    seed=10, description="B128 s_q1 h_q64 h_kv1 d128 bf16 (multi-query), s_k ~ U[1,8192]"),
}


def make_mha_inputs(batch: int, s_q: int, h_q: int, h_kv: int, head_dim: int, dtype: str = "bf16", *,
                    head_dim_v: Optional[int] = None,
                    seqlens: Optional[Sequence[int]] = None,
                    seqlen_range: Optional[tuple] = None,
                    sigma: float = 1.0, causal: bool = False, seed: int = 0,
                    extra_pages: int = 0, poison: bool = False,
                    max_pages: Optional[int] = None, kv_dtype: str = "same",
                    scale_mode: str = "amax") -> MhaInputs:
    """Seeded MHA/GQA decode inputs.  Same recipe as make_inputs, with the
    draws in the order: lengths, page permutation, q [B,s_q,h_q,d],
    k [N,64,h_kv,d], v [N,64,h_kv,d_v] (each torch.randn * sigma), then the cast
    to the dtype.  Poison (correctness runs): slots past a request's length in
    its last page and every unused page get K = +-POISON along the sign of the
    first query row of the KV head's group and V = POISON.  fp8 caches
    (kv_dtype="fp8", bf16 q): K and V are drawn and poisoned in fp32, then
    encoded per page and KV head as for the MLA cache (scale = amax / 448, or
    its power-of-two ceiling, or no scale array), scales [num_pages, h_kv]."""
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_DTYPES)}")
    if kv_dtype not in ("same", "fp8"):
        raise ValueError("kv_dtype must be 'same' or 'fp8'")
    if kv_dtype == "fp8" and dtype != "bf16":
        raise ValueError("fp8 caches go with a bf16 q")
    if h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    d_v = head_dim if head_dim_v is None else head_dim_v
    g = torch.Generator("cpu").manual_seed(int(seed))
    if seqlens is not None:
        sl = torch.tensor([int(x) for x in seqlens], dtype=torch.int64)
        if sl.numel() != batch:
            raise ValueError("len(seqlens) != batch")
    elif seqlen_range is not None:
        lo, hi = seqlen_range
        sl = torch.randint(int(lo), int(hi) + 1, (batch,), generator=g, dtype=torch.int64)
    else:
        raise ValueError("give seqlens or seqlen_range")
    n_pages = [pages_of(n) for n in sl.tolist()]
    used = sum(n_pages)
    total = used + int(extra_pages)
    perm = torch.randperm(total, generator=g) if total > 0 else torch.zeros(0, dtype=torch.int64)
    width = max(max(n_pages) if n_pages else 0, 1)
    if max_pages is not None:
        if max_pages < width:
            raise ValueError("max_pages smaller than the longest request")
        width = max_pages
    bt = torch.full((batch, width), -1, dtype=torch.int32)
    pos = 0
    for b, p in enumerate(n_pages):
        bt[b, :p] = perm[pos:pos + p].to(torch.int32)
        pos += p
    tdt = _DTYPES[dtype]
    q = (torch.randn(batch, s_q, h_q, head_dim, generator=g) * sigma).to(tdt)
    kdt = torch.float32 if kv_dtype == "fp8" else tdt
    k = (torch.randn(max(total, 1), PAGE, h_kv, head_dim, generator=g) * sigma).to(kdt)
    v = (torch.randn(max(total, 1), PAGE, h_kv, d_v, generator=g) * sigma).to(kdt)
    if poison:
        group = h_q // h_kv
        for b in range(batch):
            n = int(sl[b])
            p = pages_of(n)
            if p > 0 and n % PAGE != 0:
                page = int(bt[b, p - 1])
                for hk in range(h_kv):
                    direction = torch.sign(q[b, 0, hk * group].float())
                    direction[direction == 0] = 1.0
                    k[page, n % PAGE:, hk, :] = (direction * POISON).to(kdt)
                v[page, n % PAGE:] = POISON
        if total > used:
            k[perm[used:]] = POISON
            v[perm[used:]] = POISON
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k, k_scale = _encode_fp8_heads(k, scale_mode)
        v, v_scale = _encode_fp8_heads(v, scale_mode)
    return MhaInputs(q=q, k_cache=k, v_cache=v, block_table=bt, cache_seqlens=sl.to(torch.int32),
                     softmax_scale=1.0 / (head_dim ** 0.5), causal=causal, dtype=dtype,
                     k_scale=k_scale, v_scale=v_scale)


def _encode_fp8_heads(x: torch.Tensor, scale_mode: str):
    """fp32 cache [N, 64, h, d] -> (e4m3fn codes, scales [N, h] or None)."""
    if scale_mode == "none":
        return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn), None
    amax = x.abs().amax(dim=(1, 3)).clamp_min(1e-30)
    scale = amax / FP8_MAX
    if scale_mode == "pow2":
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    codes = (x / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale.to(torch.float32).contiguous()


def mha_workload_inputs(index: int, poison: bool = False, **overrides) -> MhaInputs:
    w = MHA_WORKLOADS[int(index)]
    kw = dict(seqlens=w.seqlens, seqlen_range=w.seqlen_range, causal=w.causal, seed=w.seed, poison=poison,
              kv_dtype=w.kv)
    kw.update(overrides)
    return make_mha_inputs(w.batch, w.s_q, w.h_q, w.h_kv, w.head_dim, w.dtype, **kw)


def workload_seqlens(index: int) -> List[int]:
    """Only the sequence lengths of a named workload (cheap: no tensors)."""
    w = WORKLOADS[int(index)] if int(index) in WORKLOADS else MHA_WORKLOADS[int(index)]
    if w.seqlens is not None:
        return list(w.seqlens)
    g = torch.Generator("cpu").manual_seed(int(w.seed))
    lo, hi = w.seqlen_range
    return torch.randint(int(lo), int(hi) + 1, (w.batch,), generator=g, dtype=torch.int64).tolist()
