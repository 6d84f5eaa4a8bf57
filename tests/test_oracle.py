"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-derived values
(tests/golden), closed forms, a pure-Python brute force, a library routine
(torch scaled_dot_product_attention in float64 on explicitly gathered rows),
and invariants (split-and-merge, page permutation).  Each pin is chosen so a
plausible slip (dropped tail mask, off-by-one causal count, wrong page lookup,
transposed operand, wrong sign or base of the scale or LSE) fails.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (D_K, D_V, PAGE, brute_force_decode, oracle_decode,
                    oracle_decode_rows, oracle_merge, oracle_partial, visible_keys)
from mla_decode_attention_02_amd.workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

_CONST = {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4), "ln6": math.log(6),
          "ln7": math.log(7), "ln66": math.log(66), "ln5/2": math.log(5) / 2,
          "ln2/3": math.log(2) / 3}


def _val(x):
    return _CONST[x] if isinstance(x, str) else float(x)


def _hand_inputs(case):
    s_q, h_q, n = case["s_q"], case["h_q"], case["seqlen"]
    pages = (n + PAGE - 1) // PAGE
    bt = np.asarray(case.get("block_table", list(range(pages))), dtype=np.int64)[None, :]
    q = np.zeros((1, s_q, h_q, D_K))
    for i, h, d, v in case["q_nonzero"]:
        q[0, i, h, d] = v
    k = np.zeros((pages, PAGE, 1, D_K))
    for j, entries in case["k_rows_nonzero"].items():
        j = int(j)
        for d, v in entries:
            k[bt[0, j // PAGE], j % PAGE, 0, d] = v
    return q, k, bt, np.asarray([n]), _val(case["scale"])


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "decode_hand_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    q, k, bt, sl, scale = _hand_inputs(case)
    out, lse = oracle_decode(q, k, bt, sl, scale, case["causal"])
    expect = np.zeros_like(out)
    for i, h, c, v in case["expect_out_nonzero"]:
        expect[0, i, h, c] = v
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-14)
    for i, h, v in case["expect_lse"]:
        assert abs(lse[0, i, h] - _val(v)) < 1e-14


def _tiny(b, s_q, h_q, seqlens, causal, seed, dtype="bf16", poison=True, extra_pages=2):
    return make_inputs(b, s_q, h_q, dtype, seqlens=seqlens, causal=causal, seed=seed,
                       poison=poison, extra_pages=extra_pages)


@pytest.mark.parametrize("s_q,h_q,seqlens,causal", [
    (1, 1, (1, 2), False),
    (1, 2, (63, 64), False),
    (2, 1, (65, 3), True),
    (2, 2, (100, 2), True),
    (1, 16, (129, 1), False),
    (2, 2, (1, 64), True),
])
def test_brute_force_matches(s_q, h_q, seqlens, causal):
    x = _tiny(len(seqlens), s_q, h_q, seqlens, causal, seed=11 + s_q * 7 + h_q)
    out, lse = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    bo, bl = brute_force_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    np.testing.assert_allclose(out, np.asarray(bo), rtol=0, atol=1e-12)
    bl = np.asarray(bl)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)


def test_single_token_returns_its_value_row():
    x = _tiny(2, 1, 4, (1, 1), False, seed=3)
    out, lse = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    k = x.k_cache.double().numpy()
    q = x.q.double().numpy()
    for b in range(2):
        row = k[int(x.block_table[b, 0]), 0, 0]
        for h in range(4):
            assert np.array_equal(out[b, 0, h], row[:D_V])         # exactly V
            s = x.softmax_scale * math.fsum(q[b, 0, h, d] * row[d] for d in range(D_K))
            assert abs(lse[b, 0, h] - s) < 1e-12                    # LSE = its score


@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (3, True), (2, False)])
def test_zero_query_gives_mean_and_log_count(s_q, causal):
    seqlens = (1, 2, 63, 64, 65, 130)
    x = _tiny(len(seqlens), s_q, 2, seqlens, causal, seed=5)
    q0 = torch.zeros_like(x.q)
    out, lse = oracle_decode(q0, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    k = x.k_cache.double().numpy()
    for b, n in enumerate(seqlens):
        rows = np.stack([k[int(x.block_table[b, j // PAGE]), j % PAGE, 0] for j in range(n)])
        for i in range(s_q):
            cnt = n - s_q + i + 1 if causal else n
            cnt = max(0, min(n, cnt))
            for h in range(2):
                if cnt == 0:
                    assert lse[b, i, h] == -math.inf and not out[b, i, h].any()
                    continue
                assert lse[b, i, h] == math.log(cnt)
                np.testing.assert_allclose(out[b, i, h], rows[:cnt, :D_V].mean(axis=0), rtol=0, atol=1e-13)


def test_equal_scores_with_distinct_value_rows():
    """q is zero on the 512 value columns and every key shares its 64 rope
    columns, so all scores are equal while the value rows differ."""
    n = 70
    x = _tiny(1, 1, 3, (n,), False, seed=8, poison=False, extra_pages=0)
    q = x.q.clone()
    q[..., :D_V] = 0
    k = x.k_cache.clone()
    k[:, :, :, D_V:] = k[0, 0, 0, D_V:]
    out, lse = oracle_decode(q, k, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    kd, qd = k.double().numpy(), q.double().numpy()
    rows = np.stack([kd[int(x.block_table[0, j // PAGE]), j % PAGE, 0] for j in range(n)])
    for h in range(3):
        s = x.softmax_scale * float(np.dot(qd[0, 0, h], rows[0]))
        np.testing.assert_allclose(out[0, 0, h], rows[:, :D_V].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, h] - (s + math.log(n))) < 1e-12


def test_dominant_key():
    n, hot = 90, 77
    x = _tiny(1, 1, 1, (n,), False, seed=9, poison=False, extra_pages=0)
    q = torch.zeros_like(x.q)
    q[0, 0, 0, 0] = 1.0
    k = x.k_cache.clone()
    k[:, :, :, 0] = 0
    page = int(x.block_table[0, hot // PAGE])
    k[page, hot % PAGE, 0, 0] = 40.0 * 24.0 / 1.0           # score gap 40 at scale 1/24
    out, lse = oracle_decode(q, k, x.block_table, x.cache_seqlens, 1.0 / 24.0, False)
    v = k[page, hot % PAGE, 0, :D_V].double().numpy()
    bound = (n - 1) * math.exp(-40.0) * (np.abs(k.double().numpy()).max() + np.abs(v).max())
    assert np.abs(out[0, 0, 0] - v).max() <= bound
    assert abs(lse[0, 0, 0] - 40.0) < 1e-12


@pytest.mark.parametrize("causal,s_q", [(False, 1), (True, 2)])
def test_split_merge_equals_unsplit(causal, s_q):
    n = 150
    x = _tiny(1, s_q, 3, (n,), causal, seed=12)
    full_o, full_l = oracle_decode_rows(x.q, x.k_cache, x.block_table, x.cache_seqlens,
                                        x.softmax_scale, causal, 0)
    for cuts in ([], [1], [64], [149], [10, 64, 128], list(range(0, 150, 17))):
        edges = [0] + [c for c in cuts if 0 < c < n] + [n]
        parts = [oracle_partial(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale,
                                causal, 0, lo, hi) for lo, hi in zip(edges[:-1], edges[1:])]
        o, l = oracle_merge(parts)
        np.testing.assert_allclose(o, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, full_l, rtol=0, atol=1e-12)


def test_merge_handles_empty_parts():
    o = np.ones((2, D_V))
    l = np.array([0.5, -np.inf])
    mo, ml = oracle_merge([(o, l), (np.zeros((2, D_V)), np.array([-np.inf, -np.inf]))])
    assert ml[0] == 0.5 and ml[1] == -np.inf
    assert np.array_equal(mo[0], o[0]) and not mo[1].any()


def test_page_permutation_is_bit_identical():
    seqlens = (200, 64, 5)
    x = _tiny(3, 2, 4, seqlens, True, seed=21)
    out1, lse1 = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    n_pages = x.k_cache.shape[0]
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(4))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n_pages)
    k2 = x.k_cache[perm]                       # new page p holds old page perm[p]
    bt2 = x.block_table.clone()
    used = bt2 >= 0
    bt2[used] = inv[bt2[used].long()].to(torch.int32)
    out2, lse2 = oracle_decode(x.q, k2, bt2, x.cache_seqlens, x.softmax_scale, True)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("causal,s_q,h_q", [(False, 1, 16), (True, 2, 8), (True, 3, 4)])
def test_matches_torch_sdpa_float64(causal, s_q, h_q):
    seqlens = (1, 64, 65, 200)
    x = _tiny(len(seqlens), s_q, h_q, seqlens, causal, seed=31 + s_q)
    out, lse = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    q = x.q.double()
    k = x.k_cache.double()
    for b, n in enumerate(seqlens):
        idx = torch.arange(n)
        rows = k[x.block_table[b, idx // PAGE].long(), idx % PAGE, 0]       # [n, 576]
        qq = q[b].reshape(s_q * h_q, D_K)
        mask = torch.zeros(s_q * h_q, n, dtype=torch.bool)
        for r in range(s_q * h_q):
            mask[r, :visible_keys(n, s_q, r // h_q, causal)] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[None, None], rows[None, None], rows[None, None, :, :D_V].contiguous(),
            attn_mask=mask[None, None], scale=x.softmax_scale)[0, 0]
        scores = (qq @ rows.T) * x.softmax_scale
        ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        live = mask.any(dim=1)
        np.testing.assert_allclose(out[b].reshape(-1, D_V)[live.numpy()], ref[live].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b].reshape(-1)[live.numpy()], ref_lse[live].numpy(), rtol=0, atol=1e-12)
        assert np.all(np.isneginf(lse[b].reshape(-1)[~live.numpy()]))


def test_empty_request_and_fully_masked_rows():
    x = _tiny(2, 3, 2, (0, 1), True, seed=2)
    out, lse = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    assert np.all(np.isneginf(lse[0])) and not out[0].any()
    # n = 1, s_q = 3: tokens 0 and 1 see nothing, token 2 sees key 0
    assert np.all(np.isneginf(lse[1, :2])) and not out[1, :2].any()
    assert np.all(np.isfinite(lse[1, 2]))


def test_poison_is_never_read():
    """Changing the poison value (slots past the length, unused pages) must not
    move a single bit of the result."""
    seqlens = (70, 130, 1)
    x = _tiny(3, 2, 2, seqlens, True, seed=40, poison=True, extra_pages=3)
    out1, lse1 = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    k = x.k_cache.clone()
    for b, n in enumerate(seqlens):
        p = (n + PAGE - 1) // PAGE
        k[int(x.block_table[b, p - 1]), n % PAGE or PAGE:, 0, :] = -7.0
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(k.shape[0]):
        if page not in used:
            k[page] = 123.0
    out2, lse2 = oracle_decode(x.q, k, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
