"""GPU parity of the paged MHA/GQA decode path (through the C ABI) against the
fp64 CPU oracle in oracle/mha.py.

Tolerances as for MLA: max |dO| <= 1.5e-2, max |dLSE| <= 1e-3; the schedule
is integer work and bit-exact.  Every case prints its name first.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import dequantize_heads, oracle_mha_decode, oracle_mha_metadata, oracle_mha_rows
from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import MHA_WORKLOADS, make_mha_inputs, mha_workload_inputs

pytestmark = pytest.mark.gpu

TOL_O = 1.5e-2
TOL_LSE = 1e-3


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


def run(x, num_parts=None):
    g = x.to(torch.device("cuda:0"))
    B, s_q, h_q, d = g.q.shape
    h_kv = g.k_cache.shape[2]
    meta = api.mha_get_metadata(g.cache_seqlens, s_q, h_q, h_kv, num_parts=num_parts)
    out, lse = api.mha_decode(g.q, g.k_cache, g.v_cache, g.block_table, g.cache_seqlens, g.softmax_scale,
                              g.causal, metadata=meta, k_scale=g.k_scale, v_scale=g.v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), [m.cpu().numpy() for m in meta]


def kv64(x):
    """K and V as the oracle sees them: exact float64 values (fp8 caches
    through the oracle's own e4m3 decoder and per-page, per-head scales)."""
    if x.k_cache.dtype == torch.float8_e4m3fn:
        return dequantize_heads(x.k_cache, x.k_scale), dequantize_heads(x.v_cache, x.v_scale)
    return x.k_cache.double().numpy(), x.v_cache.double().numpy()


def compare(out, lse, ref_o, ref_l, tag):
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse)), f"{tag}: -inf pattern differs"
    assert not np.isnan(out).any(), f"{tag}: NaN in output"
    do = np.abs(out - ref_o).max() if out.size else 0.0
    dl = np.abs(lse[fin] - ref_l[fin]).max() if fin.any() else 0.0
    assert do <= TOL_O, f"{tag}: max|dO| = {do}"
    assert dl <= TOL_LSE, f"{tag}: max|dLSE| = {dl}"
    if not fin.all():
        assert np.all(out[~fin] == 0), f"{tag}: rows with no visible key must be 0"


@pytest.mark.parametrize("seqlens,h_kv,parts", [
    ([64, 100, 0, 3000], 8, 256), ([1] * 50, 4, 7), ([131072, 5, 70000], 2, 128), ([0, 0], 3, 5),
    ([(i * 37) % 900 for i in range(3000)], 8, 256),
])
def test_mha_metadata_bit_exact(seqlens, h_kv, parts):
    _say(f"mha metadata {seqlens[:5]} h_kv={h_kv} parts={parts}")
    seq = torch.tensor(seqlens, dtype=torch.int32, device="cuda:0")
    sched, offs = api.mha_get_metadata(seq, 1, 8 * h_kv, h_kv, num_parts=parts)
    torch.cuda.synchronize()
    ref_s, ref_o = oracle_mha_metadata(seqlens, h_kv, parts)
    assert np.array_equal(sched.cpu().numpy(), ref_s)
    assert np.array_equal(offs.cpu().numpy(), ref_o)


EDGE = [
    # (s_q, h_q, h_kv, d, seqlens, causal, dtype, num_parts)
    (1, 8, 2, 128, (1, 2, 63, 64, 65), False, "bf16", None),
    (1, 8, 8, 128, (127, 128, 129, 1000), False, "fp16", 3),
    (2, 16, 2, 128, (1, 2, 65, 300), True, "bf16", 2),
    (1, 4, 1, 64, (5, 300), False, "bf16", 1),
    (3, 6, 3, 64, (300, 7, 64), True, "fp16", 5),
    (1, 32, 4, 256, (33, 64, 65, 500), False, "bf16", None),
    (2, 8, 4, 256, (1, 31, 32, 33, 97), True, "fp16", 4),
    (1, 64, 1, 128, (200, 1000), False, "bf16", 6),        # 64 rows: one full row block
    (3, 32, 1, 64, (129, 700), True, "bf16", 3),           # 96 rows: two row blocks
    (2, 40, 2, 128, (2, 129, 300), True, "bf16", 3),       # 40 rows: three row tiles
    (1, 12, 4, 128, (5000,), False, "bf16", 17),           # one long request cut into many pieces
    (1, 32, 1, 128, (70, 300), False, "fp16", 4),          # 32 rows: row split, two idle waves
    (2, 64, 2, 256, (40, 129), True, "fp16", 3),           # 64 rows, d = 256: row split, fp16
    (4, 64, 1, 128, (100, 700), True, "bf16", None),       # 256 rows: four row blocks
    (2, 128, 1, 64, (65, 300, 1), True, "bf16", 2),        # 256 rows at d = 64
    (8, 32, 1, 256, (65, 300), True, "fp16", 3),           # 256 rows at d = 256
]


@pytest.mark.parametrize("s_q,h_q,h_kv,d,seqlens,causal,dtype,parts", EDGE,
                         ids=[f"sq{c[0]}_hq{c[1]}_hkv{c[2]}_d{c[3]}_{'c' if c[5] else 'n'}_{c[6]}_p{c[7]}" for c in EDGE])
def test_mha_small_parity(s_q, h_q, h_kv, d, seqlens, causal, dtype, parts):
    tag = f"mha s_q={s_q} h_q={h_q} h_kv={h_kv} d={d} seqlens={seqlens} causal={causal} {dtype} parts={parts}"
    _say(tag)
    x = make_mha_inputs(len(seqlens), s_q, h_q, h_kv, d, dtype, seqlens=seqlens, causal=causal,
                        seed=sum(seqlens) + h_q + d, poison=True, extra_pages=2)
    out, lse, _ = run(x, parts)
    ref_o, ref_l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens,
                                     x.softmax_scale, causal)
    compare(out, lse, ref_o, ref_l, tag)


@pytest.mark.parametrize("h_q,h_kv,d,seqlens,parts,kv", [
    (8, 1, 128, (12800, 70), 150, "same"),      # ~100 pieces of one unit
    (16, 2, 64, (25600, 1), 300, "same"),       # two units of ~130 pieces each
    (8, 1, 128, (12800,), 150, "fp8"),          # the key-split kernel's pieces
], ids=["d128_100pieces", "d64_2units_130pieces", "fp8_100pieces"])
def test_mha_units_cut_into_more_than_64_pieces(h_q, h_kv, d, seqlens, parts, kv):
    _say(f"mha many pieces h_q={h_q} h_kv={h_kv} d={d} seqlens={seqlens} parts={parts} {kv}")
    x = make_mha_inputs(len(seqlens), 1, h_q, h_kv, d, "bf16", seqlens=seqlens, seed=71 + d, poison=True,
                        kv_dtype=kv)
    out, lse, meta = run(x, parts)
    assert np.diff(meta[1]).max() > 64, "expected a unit cut into more than 64 pieces"
    kf, vf = kv64(x)
    ref_o, ref_l = oracle_mha_decode(x.q, kf, vf, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    compare(out, lse, ref_o, ref_l, f"mha many pieces {kv}")


def test_mha_empty_requests_and_masked_rows():
    _say("mha empty request / fully masked causal rows")
    x = make_mha_inputs(3, 3, 8, 2, 128, "bf16", seqlens=(0, 1, 70), causal=True, seed=5, poison=True)
    out, lse, _ = run(x, 2)
    ref_o, ref_l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens,
                                     x.softmax_scale, True)
    compare(out, lse, ref_o, ref_l, "mha empty")
    assert np.all(np.isneginf(lse[0])) and not out[0].any()


def test_mha_nan_in_unused_slots_and_pages():
    """Slots past a request's length read as zeros whatever they hold (here
    NaN), and unused pages are never read: outputs equal bit for bit."""
    _say("mha NaN garbage in unused slots and pages")
    seqlens = (70, 130, 3)
    x = make_mha_inputs(3, 1, 8, 2, 128, "bf16", seqlens=seqlens, seed=23, extra_pages=3)
    out1, lse1, _ = run(x, 4)
    for b, n in enumerate(seqlens):
        page = int(x.block_table[b, (n + 63) // 64 - 1])
        x.k_cache[page, n % 64:] = float("nan")
        x.v_cache[page, n % 64:] = float("nan")
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(x.k_cache.shape[0]):
        if page not in used:
            x.k_cache[page] = float("nan")
            x.v_cache[page] = float("inf")
    out2, lse2, _ = run(x, 4)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_mha_page_permutation_is_bitwise_invariant():
    _say("mha page permutation invariance")
    x = make_mha_inputs(4, 2, 16, 4, 128, "bf16", seqlens=(300, 64, 129, 1), causal=True, seed=17, extra_pages=2)
    out1, lse1, _ = run(x, 5)
    n = x.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n)
    x.k_cache = x.k_cache[perm].contiguous()
    x.v_cache = x.v_cache[perm].contiguous()
    used = x.block_table >= 0
    x.block_table[used] = inv[x.block_table[used].long()].to(torch.int32)
    out2, lse2, _ = run(x, 5)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_mha_strided_views():
    _say("mha strided q / caches / out")
    x = make_mha_inputs(3, 1, 8, 2, 128, "bf16", seqlens=(70, 200, 5), seed=9, poison=True)
    dev = torch.device("cuda:0")
    g = x.to(dev)
    qbig = torch.zeros(3, 1, 12, 128, dtype=g.q.dtype, device=dev)
    qbig[:, :, 2:10] = g.q
    q = qbig[:, :, 2:10]
    kbig = torch.zeros(g.k_cache.shape[0], 64, 3, 128, dtype=g.q.dtype, device=dev)
    kbig[:, :, :2] = g.k_cache
    vbig = torch.zeros(g.k_cache.shape[0], 64, 2, 136, dtype=g.q.dtype, device=dev)
    vbig[..., :128] = g.v_cache
    meta = api.mha_get_metadata(g.cache_seqlens, 1, 8, 2, num_parts=3)
    bufs = api.MhaBuffers(g.q, 2, 3)
    obig = torch.zeros(3, 1, 8, 136, dtype=g.q.dtype, device=dev)
    bufs.out = obig[..., :128]
    out, lse = api.mha_decode(q, kbig[:, :, :2], vbig[..., :128], g.block_table, g.cache_seqlens, g.softmax_scale,
                              False, metadata=meta, buffers=bufs)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens,
                                     x.softmax_scale, False)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "mha strided")
    assert not obig[..., 128:].any(), "padding of the output rows was written"


@pytest.mark.parametrize("idx", sorted(MHA_WORKLOADS))
def test_mha_workload_full_size_every_request(idx):
    """Full-size GQA workload in the launch configuration the benchmark uses;
    every request is checked against the oracle (max |dO|, max |dLSE|), and
    the RMS-relative output error over the whole workload is bounded by 1e-2."""
    w = MHA_WORKLOADS[idx]
    _say(f"mha workload {idx} {w.name} full size")
    x = mha_workload_inputs(idx)
    out, lse, meta = run(x)
    qf = x.q.double().numpy()
    kf, vf = kv64(x)
    num = den = 0.0
    for b in range(w.batch):
        ref_o, ref_l = oracle_mha_rows(qf, kf, vf, x.block_table, x.cache_seqlens, x.softmax_scale, w.causal, b)
        compare(out[b], lse[b], ref_o, ref_l, f"mha workload {idx} request {b}")
        num += float(((out[b].reshape(ref_o.shape) - ref_o) ** 2).sum())
        den += float((ref_o ** 2).sum())
    rms_rel = (num / den) ** 0.5
    _say(f"mha workload {idx} rms_rel_dO = {rms_rel:.3e}")
    assert rms_rel <= 1e-2, f"mha workload {idx}: RMS-relative dO = {rms_rel}"
    assert np.isfinite(lse).all()


FP8_EDGE = [
    # (s_q, h_q, h_kv, d, seqlens, causal, scale_mode, num_parts)
    (1, 8, 2, 128, (1, 2, 63, 64, 65), False, "amax", None),
    (1, 8, 8, 128, (127, 128, 129, 1000), False, "pow2", 3),
    (2, 16, 2, 128, (1, 2, 65, 300), True, "amax", 2),
    (1, 4, 1, 64, (5, 300, 64), False, "none", 1),
    (3, 6, 3, 64, (300, 7, 64), True, "amax", 5),
    (1, 32, 4, 256, (33, 64, 65, 500), False, "amax", None),
    (2, 8, 4, 256, (1, 31, 32, 33, 97), True, "pow2", 4),
    (1, 64, 1, 128, (200, 1000), False, "amax", 6),        # 64 rows: one full row block
    (2, 40, 2, 128, (2, 129, 300), True, "amax", 3),       # 40 rows: three row tiles
    (1, 12, 4, 128, (5000,), False, "amax", 17),           # one long request cut into many pieces
    # key-split kernel with more than one row tile, and the fp8 row split at d = 256
    (1, 32, 1, 128, (70, 640, 3), False, "amax", 3),       # d=128, 32 rows: key split, two row tiles
    (1, 32, 1, 64, (65, 300), False, "pow2", None),        # d=64, 32 rows: key split, two row tiles
    (1, 48, 1, 64, (129, 64, 1), False, "amax", 4),        # d=64, 48 rows: key split, three row tiles
    (3, 32, 1, 64, (2, 129, 300), True, "amax", 3),        # d=64, 96 rows: key split, four tiles, two row blocks
    (1, 32, 1, 256, (33, 200), False, "amax", 2),          # d=256, 32 rows: fp8 row split
    (2, 16, 1, 256, (1, 65, 130), True, "none", 3),        # d=256, 32 rows, causal: fp8 row split
    (4, 64, 1, 128, (300, 9), True, "amax", None),         # 256 rows: four row blocks, fp8
]


@pytest.mark.parametrize("s_q,h_q,h_kv,d,seqlens,causal,mode,parts", FP8_EDGE,
                         ids=[f"sq{c[0]}_hq{c[1]}_hkv{c[2]}_d{c[3]}_{'c' if c[5] else 'n'}_{c[6]}_p{c[7]}"
                              for c in FP8_EDGE])
def test_mha_fp8_parity(s_q, h_q, h_kv, d, seqlens, causal, mode, parts):
    """fp8 e4m3 K/V caches with one scale per page and KV head (or none),
    against the oracle on the dequantised caches."""
    tag = f"mha fp8 s_q={s_q} h_q={h_q} h_kv={h_kv} d={d} seqlens={seqlens} causal={causal} {mode} parts={parts}"
    _say(tag)
    x = make_mha_inputs(len(seqlens), s_q, h_q, h_kv, d, "bf16", seqlens=seqlens, causal=causal,
                        seed=sum(seqlens) + 3 * h_q + d, poison=True, extra_pages=2, kv_dtype="fp8",
                        scale_mode=mode)
    out, lse, _ = run(x, parts)
    kf, vf = kv64(x)
    ref_o, ref_l = oracle_mha_decode(x.q, kf, vf, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    compare(out, lse, ref_o, ref_l, tag)


def test_mha_fp8_scales_reach_both_caches():
    """Doubling every V scale doubles O; halving every K scale and doubling
    softmax_scale changes nothing (both exact in fp32, so bit for bit)."""
    _say("mha fp8 scale propagation")
    x = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(70, 500, 9), seed=31, kv_dtype="fp8")
    out1, lse1, _ = run(x, 3)
    x2 = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(70, 500, 9), seed=31, kv_dtype="fp8")
    x2.v_scale = x2.v_scale * 2
    out2, lse2, _ = run(x2, 3)
    assert np.array_equal(lse1, lse2) and np.array_equal(out2, 2 * out1)
    x3 = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(70, 500, 9), seed=31, kv_dtype="fp8")
    x3.k_scale = x3.k_scale * 0.5
    x3.softmax_scale = x.softmax_scale * 2
    out3, lse3, _ = run(x3, 3)
    assert np.array_equal(out1, out3) and np.array_equal(lse1, lse3)


def test_mha_fp8_nan_codes_in_unused_slots_and_pages():
    """NaN codes past a request's length and in unused pages, and NaN scales
    of unused pages, change nothing: those bytes are never used."""
    _say("mha fp8 NaN codes in unused slots and pages")
    seqlens = (70, 130, 3)
    x = make_mha_inputs(3, 1, 8, 2, 128, "bf16", seqlens=seqlens, seed=29, extra_pages=3, kv_dtype="fp8")
    out1, lse1, _ = run(x, 4)
    nan8 = torch.full((1,), 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)
    for b, n in enumerate(seqlens):
        page = int(x.block_table[b, (n + 63) // 64 - 1])
        x.k_cache[page, n % 64:] = nan8
        x.v_cache[page, n % 64:] = nan8
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(x.k_cache.shape[0]):
        if page not in used:
            x.k_cache[page] = nan8
            x.v_cache[page] = nan8
            x.k_scale[page] = float("nan")
            x.v_scale[page] = float("inf")
    out2, lse2, _ = run(x, 4)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
