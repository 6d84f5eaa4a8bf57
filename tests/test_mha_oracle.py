"""Pins for the paged multi-head / grouped-query decode oracle (no GPU).

The MHA oracle is checked against the pinned MLA oracle (MLA is the case of
one KV head of width 576 whose first 512 columns are the values), against
torch's scaled_dot_product_attention in float64 on explicitly gathered and
head-expanded rows, against a pure-Python brute force, and against planted
structure (constant value rows per KV head, split-and-merge, poisoned slots),
so a wrong head mapping, page lookup, mask or merge fails.
"""

import math

import numpy as np
import pytest
import torch

from oracle import oracle_decode, oracle_merge
from oracle.mha import brute_force_mha, kv_head_of, oracle_mha_decode, oracle_mha_rows
from mla_decode_attention_02_amd.workloads import make_inputs, make_mha_inputs


def test_mla_is_the_one_latent_head_case():
    x = make_inputs(3, 2, 5, "bf16", seqlens=(130, 1, 64), causal=True, seed=3, extra_pages=1)
    k = x.k_cache
    v = k[..., :512]
    o1, l1 = oracle_mha_decode(x.q, k, v, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    o2, l2 = oracle_decode(x.q, k, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def _sdpa_reference(x):
    q = x.q.double()
    B, s_q, h_q, d = q.shape
    h_kv = x.k_cache.shape[2]
    outs = torch.zeros(B, s_q, h_q, x.v_cache.shape[-1], dtype=torch.float64)
    lses = torch.full((B, s_q, h_q), -math.inf, dtype=torch.float64)
    for b in range(B):
        n = int(x.cache_seqlens[b])
        if n == 0:
            continue
        pages = x.block_table[b, :(n + 63) // 64].long()
        K = x.k_cache[pages].double().reshape(-1, h_kv, d)[:n]             # [n, h_kv, d]
        V = x.v_cache[pages].double().reshape(-1, h_kv, x.v_cache.shape[-1])[:n]
        K = K.repeat_interleave(h_q // h_kv, dim=1).transpose(0, 1)          # [h_q, n, d]
        V = V.repeat_interleave(h_q // h_kv, dim=1).transpose(0, 1)
        Q = q[b].transpose(0, 1)                                            # [h_q, s_q, d]
        i = torch.arange(s_q)[:, None]
        j = torch.arange(n)[None, :]
        mask = (j <= n - s_q + i) if x.causal else torch.ones(s_q, n, dtype=torch.bool)
        rows = mask.any(dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q[:, rows], K.contiguous(), V.contiguous(), attn_mask=mask[rows], scale=x.softmax_scale)
        outs[b, rows] = o.transpose(0, 1)
        S = (Q[:, rows] @ K.transpose(1, 2)) * x.softmax_scale
        S = S.masked_fill(~mask[rows], -math.inf)
        lses[b, rows] = torch.logsumexp(S, dim=-1).transpose(0, 1)
    return outs.numpy(), lses.numpy()


@pytest.mark.parametrize("s_q,h_q,h_kv,d,dv,causal", [
    (1, 8, 2, 64, 64, False), (2, 4, 4, 128, 128, True), (3, 6, 1, 32, 48, True), (1, 16, 8, 128, 128, False),
])
def test_matches_torch_sdpa_float64(s_q, h_q, h_kv, d, dv, causal):
    x = make_mha_inputs(4, s_q, h_q, h_kv, d, "bf16", head_dim_v=dv, seqlens=(1, 65, 200, 2), causal=causal,
                        seed=11 + d, extra_pages=2)
    o, l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    ro, rl = _sdpa_reference(x)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l))
    np.testing.assert_allclose(l[fin], rl[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(causal):
    x = make_mha_inputs(2, 2, 4, 2, 8, "fp16", head_dim_v=6, seqlens=(67, 3), causal=causal, seed=5)
    o, l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    bo, bl = brute_force_mha(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=0, atol=1e-12)


def test_kv_head_mapping_by_planted_values():
    h_q, h_kv = 6, 3
    x = make_mha_inputs(2, 1, h_q, h_kv, 16, "bf16", seqlens=(100, 7), seed=9)
    for hk in range(h_kv):
        x.v_cache[:, :, hk, :] = float(hk + 2)
    o, l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    for h in range(h_q):
        assert kv_head_of(h, h_q, h_kv) == h // 2
        np.testing.assert_allclose(o[:, :, h, :], float(h // 2 + 2), rtol=0, atol=1e-12)
    # changing KV head 2 leaves heads 0..3 unchanged, bit for bit
    x.k_cache[:, :, 2, :] *= -3.0
    o2, l2 = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    assert np.array_equal(o2[:, :, :4], o[:, :, :4]) and np.array_equal(l2[:, :, :4], l[:, :, :4])
    assert not np.array_equal(l2[:, :, 4:], l[:, :, 4:])


def test_split_and_merge_equals_whole():
    x = make_mha_inputs(1, 2, 4, 2, 32, "bf16", seqlens=(300,), causal=True, seed=13)
    whole = oracle_mha_rows(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True, 0)
    for cuts in ((0, 64, 300), (0, 1, 129, 256, 300), (0, 299, 300)):
        parts = [oracle_mha_rows(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale,
                                 True, 0, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        flat = [(o.reshape(-1, o.shape[-1]), l.reshape(-1)) for o, l in parts]
        mo, ml = oracle_merge(flat)
        np.testing.assert_allclose(mo, whole[0].reshape(-1, 32), rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, whole[1].reshape(-1), rtol=0, atol=1e-12)


def test_empty_and_fully_masked_rows():
    x = make_mha_inputs(2, 3, 2, 1, 16, "bf16", seqlens=(0, 1), causal=True, seed=2)
    o, l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    assert np.all(np.isneginf(l[0])) and not o[0].any()
    assert np.all(np.isneginf(l[1, :2])) and not o[1, :2].any()     # tokens 0, 1 see no key
    assert np.isfinite(l[1, 2]).all()


def test_poisoned_slots_are_never_read():
    kw = dict(seqlens=(70, 130, 3), seed=21, extra_pages=3)
    clean = make_mha_inputs(3, 1, 8, 4, 32, "bf16", **kw)
    dirty = make_mha_inputs(3, 1, 8, 4, 32, "bf16", poison=True, **kw)
    assert not torch.equal(clean.k_cache, dirty.k_cache)
    a = oracle_mha_decode(clean.q, clean.k_cache, clean.v_cache, clean.block_table, clean.cache_seqlens,
                          clean.softmax_scale, False)
    b = oracle_mha_decode(dirty.q, dirty.k_cache, dirty.v_cache, dirty.block_table, dirty.cache_seqlens,
                          dirty.softmax_scale, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_uneven_groups():
    with pytest.raises(ValueError):
        make_mha_inputs(1, 1, 6, 4, 16, seqlens=(3,))


def test_unit_schedule_is_the_request_schedule_of_the_repeated_lengths():
    from oracle import oracle_metadata, oracle_mha_metadata

    seqlens = [5, 0, 300, 64]
    s1, o1 = oracle_mha_metadata(seqlens, 3, 7)
    s2, o2 = oracle_metadata([5, 5, 5, 0, 0, 0, 300, 300, 300, 64, 64, 64], 7)
    assert np.array_equal(s1, s2) and np.array_equal(o1, o2)
    assert o1.shape == (13,)


def test_fp8_heads_scale_per_page_and_head():
    from oracle import decode_e4m3fn, dequantize_heads

    codes = np.full((3, 64, 2, 8), 0x38, dtype=np.uint8)      # every value 1.0
    scale = np.array([[0.5, 2.0], [3.0, 0.25], [1.0, 7.0]], dtype=np.float32)
    x = dequantize_heads(codes, scale)
    for p_ in range(3):
        for h in range(2):
            assert np.all(x[p_, :, h, :] == float(scale[p_, h]))
    assert np.array_equal(dequantize_heads(codes, None), decode_e4m3fn(codes))
    with pytest.raises(ValueError):
        dequantize_heads(codes, scale[:, :1])


@pytest.mark.parametrize("mode", ["amax", "pow2", "none"])
def test_fp8_mha_generator_within_rounding(mode):
    from oracle import dequantize_heads

    kw = dict(seqlens=(100, 3), seed=5, extra_pages=1)
    x8 = make_mha_inputs(2, 1, 8, 2, 64, "bf16", kv_dtype="fp8", scale_mode=mode, **kw)
    xb = make_mha_inputs(2, 1, 8, 2, 64, "bf16", **kw)
    assert torch.equal(x8.q, xb.q)
    for c8, s8, cb in ((x8.k_cache, x8.k_scale, xb.k_cache), (x8.v_cache, x8.v_scale, xb.v_cache)):
        vals = dequantize_heads(c8, s8)
        ref = cb.double().numpy()
        s = np.ones((vals.shape[0], vals.shape[2])) if s8 is None else s8.double().numpy()
        bound = (2.0 ** -4 + 2.0 ** -8) * np.abs(ref) + s[:, None, :, None] * 2.0 ** -9
        assert np.all(np.abs(vals - ref) <= bound)
