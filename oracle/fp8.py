"""fp8 e4m3 codes of a latent KV cache -> exact values (fp64 CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (page title, then section):
  [RUIBAO-FP8]   "DeepSeek开源FlashMLA全解析：性能革命背后的技术密码", section
                 "1.2 计算模式创新：混合精度矩阵乘法": the query-key product is
                 formed from fp8 values while the softmax and the value product
                 stay in 16-bit floats.
  [LITE-FP8]     "云上AI推理新突破：FlashMLA赋能DeepSeek-V2-Lite提速16%", section
                 "3. 动态精度缩放": the same split, with fp8 casts of q and k.

Reading (listed in the design notes): the pages name fp8 for the key side but
fix neither the encoding nor a scale.  Here the cached latent rows are stored
as fp8 codes in the OCP e4m3 "fn" encoding (1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 is subnormal; no infinities; the two
codes with every exponent and mantissa bit set are NaN) with one fp32 scale
per 64-token page: the cached value is code value * scale[page].  q stays bf16
and the attention is the one of decode.py over those values.  For the separate
K and V caches of the multi-head path (mha.py) the same encoding carries one
scale per page and KV head (dequantize_heads).
"""

from __future__ import annotations

import math

import numpy as np

EXP_BIAS = 7
MAN_BITS = 3


def e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn byte, from the bit fields (pure Python)."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("an fp8 code is one byte")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> MAN_BITS) & 0xF
    m = code & ((1 << MAN_BITS) - 1)
    if e == 0xF and m == (1 << MAN_BITS) - 1:
        return math.nan
    if e == 0:                                  # subnormal: m/8 * 2^(1-bias)
        return sign * math.ldexp(m, 1 - EXP_BIAS - MAN_BITS)
    return sign * math.ldexp((1 << MAN_BITS) + m, e - EXP_BIAS - MAN_BITS)


def _table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_VALUES = _table()


def decode_e4m3fn(codes) -> np.ndarray:
    """Array of e4m3fn codes (uint8, or a torch float8_e4m3fn / uint8 tensor)
    -> float64 values of the same shape."""
    try:
        import torch

        if isinstance(codes, torch.Tensor):
            if codes.dtype != torch.uint8:
                codes = codes.view(torch.uint8)
            codes = codes.detach().cpu().numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise ValueError("codes must be uint8")
    return _VALUES[codes]


def dequantize_cache(codes, k_scale=None) -> np.ndarray:
    """fp8 cache [num_pages, 64, h_kv, 576] of codes and its per-page scales
    [num_pages] (None: every scale is 1) -> float64 cache of the same shape
    holding code value * scale[page]."""
    v = decode_e4m3fn(codes)
    if k_scale is None:
        return v
    try:
        import torch

        if isinstance(k_scale, torch.Tensor):
            k_scale = k_scale.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    s = np.asarray(k_scale, dtype=np.float64)
    if s.shape != (v.shape[0],):
        raise ValueError("k_scale must hold one scale per page")
    return v * s.reshape((-1,) + (1,) * (v.ndim - 1))


def dequantize_heads(codes, scale=None) -> np.ndarray:
    """fp8 cache [num_pages, 64, h_kv, d] of codes and scales [num_pages, h_kv]
    (one per page and KV head; None: every scale is 1) -> float64 cache of the
    same shape holding code value * scale[page, head]."""
    v = decode_e4m3fn(codes)
    if scale is None:
        return v
    try:
        import torch

        if isinstance(scale, torch.Tensor):
            scale = scale.detach().cpu().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    s = np.asarray(scale, dtype=np.float64)
    if s.shape != (v.shape[0], v.shape[2]):
        raise ValueError("scale must hold one value per page and KV head")
    return v * s[:, None, :, None]


# ------------------------------------------------- fp8 query quantization --
# [RUIBAO-FP8] and [LITE-FP8] also take the query into fp8 for the query-key
# product.  Reading: each query row (one token of one head, its 576 values) is
# quantized on its own: with a = max |q| over the row, the scale is the power
# of two 2^k with the smallest k such that a * 2^-k <= 448 (the largest e4m3
# value; k = 0 for a row of zeros), and each value becomes the e4m3 code
# nearest to q * 2^-k, ties to the code with an even last mantissa bit.  The
# scaling is exact, so the rounding to e4m3 is the only one.  The product is
# then the attention of decode.py with q replaced by code value * 2^k.

E4M3_MAX = 448.0
_FINITE = np.array(sorted({abs(v) for v in _VALUES if not math.isnan(v)}), dtype=np.float64)   # 0 .. 448
_FINITE_CODE = np.array([next(c for c in range(128) if _VALUES[c] == v) for v in _FINITE], dtype=np.uint8)


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code to each float with |x| <= 448 (ties to the even
    code); uint8 array of x's shape.  A value that rounds to zero keeps its
    sign in the code (0x80 for negative values)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("values must be finite and within +-448")
    a = np.abs(x)
    hi = np.searchsorted(_FINITE, a, side="left")          # first representable >= a
    lo = np.maximum(hi - 1, 0)
    hi = np.minimum(hi, len(_FINITE) - 1)
    dlo, dhi = a - _FINITE[lo], _FINITE[hi] - a
    c_lo, c_hi = _FINITE_CODE[lo], _FINITE_CODE[hi]
    take_hi = (dhi < dlo) | ((dhi == dlo) & (c_hi % 2 == 0) & (c_lo % 2 == 1))
    code = np.where(take_hi, c_hi, c_lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def row_scale_exponent(a: float) -> int:
    """The k of the query row scale 2^k for a row maximum a >= 0 (see above)."""
    if a == 0.0:
        return 0
    _, e = math.frexp(a)                   # a = f * 2^e, f in [0.5, 1)
    k = e - 9                              # a * 2^-k in [256, 512)
    if math.ldexp(a, -k) > E4M3_MAX:
        k += 1
    assert math.ldexp(a, -k) <= E4M3_MAX < math.ldexp(a, -(k - 1))
    return k


def quantize_q_rows(q) -> np.ndarray:
    """q [..., 576] (bf16/fp16 tensor or array) -> the float64 values the fp8
    query-key product uses: code value * 2^k, one k per row."""
    try:
        import torch

        if isinstance(q, torch.Tensor):
            q = q.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    q = np.asarray(q, dtype=np.float64)
    rows = q.reshape(-1, q.shape[-1])
    out = np.empty_like(rows)
    for i, r in enumerate(rows):
        k = row_scale_exponent(float(np.abs(r).max()) if r.size else 0.0)
        out[i] = decode_e4m3fn(encode_e4m3fn(np.ldexp(r, -k))) * math.ldexp(1.0, k)
    return out.reshape(q.shape)
