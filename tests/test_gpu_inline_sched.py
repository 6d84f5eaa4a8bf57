"""GPU: decode calls that pass no schedule.  The split-KV and combine kernels
then evaluate the scheduler's rule themselves from cache_seqlens; the pieces,
their slots and hence every output bit must equal those of the same call with
the schedule precomputed by mla_get_metadata (itself bit-exact against the
oracle's schedule in test_gpu_parity.py).  One case per kernel family is also
checked against the fp64 oracle directly.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import dequantize_cache, oracle_decode
from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    yield
    torch.cuda.synchronize()


def _mixed(batch, seed):
    """Lengths with empty requests, single tokens, page edges and long ones."""
    rng = np.random.default_rng(seed)
    pool = [0, 1, 63, 64, 65, 127, 128, 129, 700, 2000, 4097]
    return [int(pool[i % len(pool)]) if i % 3 else int(rng.integers(0, 3000)) for i in range(batch)]


# (tag, batch, s_q, h_q, dtype, kv, causal, seqlens, num_parts)
CASES = [
    ("narrow bf16", 7, 1, 16, "bf16", "same", False, None, None),
    ("narrow fp16 causal s_q=2", 5, 2, 8, "fp16", "same", True, None, 3),
    ("narrow bf16 one part", 4, 1, 16, "bf16", "same", False, None, 1),
    ("narrow fp8", 9, 1, 16, "bf16", "fp8", False, None, 17),
    ("wide bf16", 6, 1, 128, "bf16", "same", False, None, None),
    ("wide bf16 causal s_q=2", 4, 2, 64, "bf16", "same", True, None, 5),
    ("wide fp8", 5, 1, 128, "bf16", "fp8", False, None, 7),
    ("300 requests (two length blocks)", 300, 1, 16, "bf16", "same", False, "short", 64),
    ("600 requests, few parts", 600, 1, 16, "fp16", "same", False, "short", 3),
    ("all empty", 4, 1, 16, "bf16", "same", False, [0, 0, 0, 0], 8),
    ("over 64 pieces, half rows", 2, 1, 16, "bf16", "same", False, [9000, 8000], 200),
    ("over 64 pieces, whole rows", 64, 1, 64, "bf16", "same", False, [40000] + [64] * 63, 256),
]


def _inputs(batch, s_q, h_q, dtype, kv, causal, seqlens, seed):
    if seqlens is None:
        seqlens = _mixed(batch, seed)
    elif seqlens == "short":
        rng = np.random.default_rng(seed)
        seqlens = [int(v) for v in rng.integers(0, 200, size=batch)]
    if causal:
        seqlens = [max(v, s_q) for v in seqlens]
    return make_inputs(batch, s_q, h_q, dtype, seqlens=tuple(seqlens), causal=causal, seed=seed, poison=True,
                       kv_dtype=kv)


def _decode(entry, g, meta, parts):
    if entry == "mla_decode_noalloc":
        return api.mla_decode_noalloc(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, g.causal,
                                      metadata=meta, k_scale=g.k_scale)
    bufs = api.DecodeBuffers(g.q, parts)
    return getattr(api, entry)(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, g.causal,
                               metadata=meta, buffers=bufs, k_scale=g.k_scale)


@pytest.mark.parametrize("entry", ["mla_decode", "mla_decode_fused", "mla_decode_noalloc"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_inline_schedule_matches_precomputed(case, entry):
    tag, batch, s_q, h_q, dtype, kv, causal, seqlens, parts = case
    _say(f"inline schedule: {tag} via {entry}")
    x = _inputs(batch, s_q, h_q, dtype, kv, causal, seqlens, seed=batch * 31 + h_q)
    g = x.to(torch.device("cuda:0"))
    if parts is None:
        parts = api.get_metadata_shape(batch, s_q, h_q)[0]
    meta = api.get_metadata(g.cache_seqlens, s_q, h_q, num_parts=parts)
    o_pre, l_pre = _decode(entry, g, meta, parts)
    o_pre, l_pre = o_pre.clone(), l_pre.clone()
    o_in, l_in = _decode(entry, g, parts, parts)
    torch.cuda.synchronize()
    assert torch.equal(o_in, o_pre), f"{tag}: outputs differ from the precomputed schedule's"
    assert torch.equal(l_in, l_pre), f"{tag}: LSEs differ from the precomputed schedule's"


@pytest.mark.parametrize("h_q,kv", [(16, "same"), (16, "fp8"), (128, "same"), (128, "fp8")])
def test_inline_schedule_against_oracle(h_q, kv):
    _say(f"inline schedule vs oracle: h_q={h_q} kv={kv}")
    x = _inputs(6, 1, h_q, "bf16", kv, False, None, seed=77 + h_q)
    g = x.to(torch.device("cuda:0"))
    out, lse = api.mla_decode(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, False,
                              k_scale=g.k_scale)          # no metadata: the in-kernel schedule
    torch.cuda.synchronize()
    cache = dequantize_cache(x.k_cache, x.k_scale) if kv == "fp8" else x.k_cache.double().numpy()
    ref_o, ref_l = oracle_decode(x.q, cache, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(out - ref_o).max() <= 1.5e-2
    assert np.abs(lse[fin] - ref_l[fin]).max() <= 1e-3


# ------------------------------------------------------------- MHA path --
# (tag, batch, s_q, h_q, h_kv, d, kv, causal, num_parts)
MHA_CASES = [
    ("gqa d128", 6, 1, 8, 2, 128, "same", False, None),
    ("gqa d64 causal s_q=2", 5, 2, 8, 4, 64, "same", True, 7),
    ("gqa d256", 3, 1, 4, 1, 256, "same", False, 5),
    ("mqa 32 heads (row split)", 4, 1, 32, 1, 128, "same", False, None),
    ("gqa fp8 K/V (key split)", 6, 1, 8, 2, 128, "fp8", False, 11),
    ("300 units", 150, 1, 4, 2, 64, "same", False, 64),
]


@pytest.mark.parametrize("case", MHA_CASES, ids=[c[0] for c in MHA_CASES])
def test_mha_inline_schedule_matches_precomputed(case):
    from mla_decode_attention_02_amd.workloads import make_mha_inputs

    tag, batch, s_q, h_q, h_kv, d, kv, causal, parts = case
    _say(f"inline schedule, MHA: {tag}")
    seqlens = _mixed(batch, seed=batch + d)
    if causal:
        seqlens = [max(v, s_q) for v in seqlens]
    x = make_mha_inputs(batch, s_q, h_q, h_kv, d, "bf16", seqlens=tuple(seqlens), causal=causal, seed=batch * 7 + d,
                        poison=True, kv_dtype=kv)
    g = x.to(torch.device("cuda:0"))
    if parts is None:
        parts = api.mha_get_metadata_shape(batch, s_q, h_q, h_kv)[0]
    meta = api.mha_get_metadata(g.cache_seqlens, s_q, h_q, h_kv, num_parts=parts)
    outs = []
    for m in (meta, parts):
        bufs = api.MhaBuffers(g.q, h_kv, parts)
        o, l = api.mha_decode(g.q, g.k_cache, g.v_cache, g.block_table, g.cache_seqlens, g.softmax_scale, causal,
                              metadata=m, buffers=bufs, k_scale=g.k_scale, v_scale=g.v_scale)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]), f"{tag}: outputs differ from the precomputed schedule's"
    assert torch.equal(outs[0][1], outs[1][1]), f"{tag}: LSEs differ from the precomputed schedule's"
