"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (bf16/fp16 inputs, fp32 accumulation): max |dO| <= 1.5e-2 and
max |dLSE| <= 1e-3 against the oracle on the same seeded inputs, and at full
size an RMS-relative output error <= 1e-2 over the whole workload; the
schedule is integer work and must be bit-exact.  Every case prints its name first so a
failing run identifies itself.
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import dequantize_cache, oracle_decode, oracle_decode_rows, oracle_metadata
from oracle.fp8 import quantize_q_rows
from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import WORKLOADS, make_inputs, workload_inputs, workload_seqlens

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


ENTRIES = ["mla_decode", "mla_decode_fused"]


def run(x, num_parts=None, entry="mla_decode", buffers=None, qk_fp8=False):
    dev = torch.device("cuda:0")
    g = x.to(dev)
    meta = api.get_metadata(g.cache_seqlens, g.q.shape[1], g.q.shape[2], num_parts=num_parts)
    out, lse = getattr(api, entry)(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale,
                                   g.causal, metadata=meta, buffers=buffers, k_scale=g.k_scale, qk_fp8=qk_fp8)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), [m.cpu().numpy() for m in meta]


def kv64(x):
    """The cache as the oracle sees it: exact values in float64 (an fp8 cache
    through the oracle's own e4m3 decoder and page scales)."""
    if x.k_cache.dtype == torch.float8_e4m3fn:
        return dequantize_cache(x.k_cache, x.k_scale)
    return x.k_cache.double().numpy()


def compare(out, lse, ref_o, ref_l, tag, tol_o=TOL_O):
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse)), f"{tag}: -inf pattern differs"
    assert not np.isnan(out).any(), f"{tag}: NaN in output"
    do = np.abs(out - ref_o).max() if out.size else 0.0
    dl = np.abs(lse[fin] - ref_l[fin]).max() if fin.any() else 0.0
    assert do <= tol_o, f"{tag}: max|dO| = {do}"
    assert dl <= TOL_LSE, f"{tag}: max|dLSE| = {dl}"
    if not fin.all():
        assert np.all(out[~fin] == 0), f"{tag}: rows with no visible key must be 0"
    return do, dl


# ------------------------------------------------------------- schedule --
@pytest.mark.parametrize("seqlens,parts", [
    ([64, 100], 256),
    ([640, 192, 0, 65], 3),
    ([1280], 4),
    ([100, 1000, 1], 2),
    ([0, 0, 0], 5),
    ([1] * 300, 7),
    ([131072, 1, 2, 3, 70000], 128),
    ([(i * 37) % 900 for i in range(9000)], 256),
    ([(i * 53) % 300 for i in range(20000)], 256),   # beyond the scheduler's LDS staging
])
def test_metadata_bit_exact(seqlens, parts):
    _say(f"metadata {seqlens[:6]} parts={parts}")
    seq = torch.tensor(seqlens, dtype=torch.int32, device="cuda:0")
    sched, offs = api.get_metadata(seq, 1, 16, num_parts=parts)
    torch.cuda.synchronize()
    ref_s, ref_o = oracle_metadata(seqlens, parts)
    assert np.array_equal(sched.cpu().numpy(), ref_s)
    assert np.array_equal(offs.cpu().numpy(), ref_o)


@pytest.mark.parametrize("F", [0, 1, 4, 9, 64])
@pytest.mark.parametrize("seqlens,parts", [
    ([640, 192, 0, 65], 3),
    ([(i * 37) % 900 for i in range(9000)], 256),
    ([(i * 53) % 300 for i in range(20000)], 256),   # beyond the scheduler's LDS staging
], ids=["small", "9000", "20000"])
def test_metadata_explicit_overhead_bit_exact(seqlens, parts, F):
    _say(f"metadata F={F} batch={len(seqlens)} parts={parts}")
    seq = torch.tensor(seqlens, dtype=torch.int32, device="cuda:0")
    sched, offs = api.get_metadata(seq, 1, 16, num_parts=parts, fixed_overhead=F)
    torch.cuda.synchronize()
    ref_s, ref_o = oracle_metadata(seqlens, parts, fixed_overhead=F)
    assert np.array_equal(sched.cpu().numpy(), ref_s)
    assert np.array_equal(offs.cpu().numpy(), ref_o)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6, 11, 12])
def test_metadata_workloads_bit_exact(idx):
    w = WORKLOADS[idx]
    seqlens = workload_seqlens(idx)
    seq = torch.tensor(seqlens, dtype=torch.int32, device="cuda:0")
    sched, offs = api.get_metadata(seq, w.s_q, w.h_q)
    torch.cuda.synchronize()
    parts = sched.shape[0]
    _say(f"metadata workload {idx} parts={parts}")
    ref_s, ref_o = oracle_metadata(seqlens, parts)
    assert np.array_equal(sched.cpu().numpy(), ref_s)
    assert np.array_equal(offs.cpu().numpy(), ref_o)


# --------------------------------------------------------- small parity --
EDGE = [
    # (s_q, h_q, seqlens, causal, dtype, num_parts)
    (1, 16, (1, 2, 63, 64, 65), False, "bf16", None),
    (1, 16, (127, 128, 129, 1000), False, "fp16", 3),
    (2, 8, (1, 2, 63, 64, 65, 129), True, "bf16", 2),
    (1, 1, (5, 300), False, "bf16", 1),
    (1, 3, (300, 7), False, "fp16", 5),
    (1, 64, (1, 64, 65, 200), False, "bf16", None),
    (1, 64, (127, 640), False, "bf16", 4),
    (2, 32, (1, 2, 65, 300), True, "fp16", 3),
    (1, 128, (129, 1000), False, "bf16", 7),
    (2, 128, (2, 3, 700), True, "fp16", 2),
    (3, 40, (2, 129, 300), True, "bf16", 3),
    (1, 17, (500, 64), False, "bf16", 6),
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("s_q,h_q,seqlens,causal,dtype,parts", EDGE,
                         ids=[f"sq{c[0]}_hq{c[1]}_{'c' if c[3] else 'n'}_{c[4]}_p{c[5]}" for c in EDGE])
def test_small_parity(s_q, h_q, seqlens, causal, dtype, parts, entry):
    tag = f"small {entry} s_q={s_q} h_q={h_q} seqlens={seqlens} causal={causal} {dtype} parts={parts}"
    _say(tag)
    x = make_inputs(len(seqlens), s_q, h_q, dtype, seqlens=seqlens, causal=causal,
                    seed=sum(seqlens) + h_q, poison=True, extra_pages=3)
    out, lse, _ = run(x, parts, entry)
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    compare(out, lse, ref_o, ref_l, tag)


# Many row tiles per request: s_q * h_q of 512 to 1024 rows (8 to 16 tiles of
# 64, so the default partition count falls to 32 or 16 per tile), causal and
# not, with ragged lengths; the fp8 cache and the fp8 query-key product too.
MANY_ROWS = [
    # (s_q, h_q, seqlens, causal, dtype, kv, qk8, num_parts)
    (4, 128, (100, 700), True, "bf16", "same", False, None),
    (8, 128, (65, 300), True, "fp16", "same", False, 3),
    (6, 100, (129,), False, "bf16", "same", False, 2),
    (4, 128, (200, 9, 64), True, "bf16", "fp8", False, None),
    (4, 128, (300, 1), True, "bf16", "fp8", True, 5),
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("s_q,h_q,seqlens,causal,dtype,kv,qk8,parts", MANY_ROWS,
                         ids=[f"sq{c[0]}_hq{c[1]}_{c[5]}{'_qk8' if c[6] else ''}_p{c[7]}" for c in MANY_ROWS])
def test_many_row_tiles(s_q, h_q, seqlens, causal, dtype, kv, qk8, parts, entry):
    tag = f"many rows {entry} s_q={s_q} h_q={h_q} seqlens={seqlens} causal={causal} {dtype} {kv} qk8={qk8} parts={parts}"
    _say(tag)
    x = make_inputs(len(seqlens), s_q, h_q, dtype, seqlens=seqlens, causal=causal,
                    seed=sum(seqlens) + s_q * h_q, poison=True, extra_pages=2, kv_dtype=kv)
    out, lse, _ = run(x, parts, entry, qk_fp8=qk8)
    if qk8:
        q = quantize_q_rows(x.q)
    else:
        q = x.q
    ref_o, ref_l = oracle_decode(q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    compare(out, lse, ref_o, ref_l, tag)


@pytest.mark.parametrize("entry", ENTRIES)
def test_empty_request_and_masked_rows(entry):
    _say(f"empty request / fully masked causal rows ({entry})")
    x = make_inputs(3, 3, 16, "bf16", seqlens=(0, 1, 70), causal=True, seed=5, poison=True)
    out, lse, _ = run(x, 2, entry)
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, True)
    compare(out, lse, ref_o, ref_l, "empty")
    assert np.all(np.isneginf(lse[0])) and not out[0].any()


def test_workload1_tiny_full():
    _say("workload 1 (tiny), full comparison")
    x = workload_inputs(1, poison=True)
    out, lse, _ = run(x)
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, x.causal)
    compare(out, lse, ref_o, ref_l, "workload 1")


def test_strided_views():
    _say("strided q / k_cache / out views")
    x = make_inputs(3, 1, 64, "bf16", seqlens=(70, 200, 5), seed=9, poison=True)
    dev = torch.device("cuda:0")
    g = x.to(dev)
    # q as a head-slice of a wider tensor, k_cache with padded slots
    qbig = torch.zeros(3, 1, 80, 576, dtype=g.q.dtype, device=dev)
    qbig[:, :, 8:72] = g.q
    q = qbig[:, :, 8:72]
    kbig = torch.zeros(g.k_cache.shape[0], 64, 1, 640, dtype=g.k_cache.dtype, device=dev)
    kbig[..., :576] = g.k_cache
    k = kbig[..., :576]
    meta = api.get_metadata(g.cache_seqlens, 1, 64, num_parts=3)
    bufs = api.DecodeBuffers(g.q, 3)
    obig = torch.zeros(3, 1, 64, 520, dtype=g.q.dtype, device=dev)
    bufs.out = obig[..., :512]
    out, lse = api.mla_decode(q, k, g.block_table, g.cache_seqlens, g.softmax_scale, False,
                              metadata=meta, buffers=bufs)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "strided")
    assert not obig[..., 512:].any(), "padding of the output rows was written"


# ------------------------------------------------------------ fp8 cache --
FP8_EDGE = [
    # (s_q, h_q, seqlens, causal, scale_mode, num_parts)
    (1, 16, (1, 2, 63, 64, 65), False, "amax", None),
    (1, 16, (127, 128, 129, 1000), False, "pow2", 3),
    (2, 8, (1, 2, 63, 64, 65, 129), True, "amax", 2),
    (1, 1, (5, 300), False, "none", 1),
    (1, 3, (300, 7), False, "amax", 5),
    (4, 4, (3, 200, 64), True, "pow2", 4),
    (1, 16, (2000, 1, 700), False, "amax", 9),
    # more than 16 rows: 64-row tiles
    (1, 128, (1, 63, 64, 65, 300), False, "amax", None),
    (2, 64, (1, 2, 64, 129, 500), True, "pow2", 3),
    (1, 32, (700, 5), False, "none", 4),
    (1, 128, (2000,), False, "amax", 7),
    (3, 40, (100, 1, 333), True, "amax", 2),
    (1, 17, (129, 64, 31), False, "pow2", None),
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("s_q,h_q,seqlens,causal,mode,parts", FP8_EDGE,
                         ids=[f"sq{c[0]}_hq{c[1]}_{'c' if c[3] else 'n'}_{c[4]}_p{c[5]}" for c in FP8_EDGE])
def test_fp8_small_parity(s_q, h_q, seqlens, causal, mode, parts, entry):
    tag = f"fp8 {entry} s_q={s_q} h_q={h_q} seqlens={seqlens} causal={causal} scale={mode} parts={parts}"
    _say(tag)
    x = make_inputs(len(seqlens), s_q, h_q, "bf16", seqlens=seqlens, causal=causal, seed=sum(seqlens) + 7 * h_q,
                    poison=True, extra_pages=2, kv_dtype="fp8", scale_mode=mode)
    out, lse, _ = run(x, parts, entry)
    ref_o, ref_l = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    compare(out, lse, ref_o, ref_l, tag)


def range_tol(ref_o):
    """Output bound when a page scale makes the outputs large: the bf16
    rounding of the output and of the probabilities is 2^-8 relative each, on
    values up to the largest output, so together about 2^-7 max|O|; TOL_O is
    that for max|O| = 2, and the bound grows in proportion beyond it."""
    return TOL_O * max(1.0, float(np.abs(ref_o).max()) / 2.0)


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_scale_is_applied_per_page(h_q):
    """One used page's scale is tripled: the result must follow the oracle, which
    a kernel that ignored the scale, or took another page's, would not (the
    two oracle results differ by several units).  That page's values, and so
    the outputs and their bf16 rounding step, grow up to threefold: the output
    tolerance grows with the largest oracle output."""
    _say(f"fp8 per-page scale h_q={h_q}")
    x = make_inputs(2, 1, h_q, "bf16", seqlens=(300, 129), seed=77, kv_dtype="fp8")
    before, _ = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, False)
    x.k_scale[int(x.block_table[0, 2])] *= 3.0
    out, lse, _ = run(x, 3)
    ref_o, ref_l = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, False)
    assert np.abs(ref_o - before).max() > 1.0
    compare(out, lse, ref_o, ref_l, "fp8 page scale x3", tol_o=range_tol(ref_o))


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_negative_and_zero_scales(h_q):
    """Any finite scale is allowed: one page's scale made negative (its keys
    and values change sign), another's zero (its keys score 0 and its values
    vanish)."""
    _say(f"fp8 negative and zero scales h_q={h_q}")
    x = make_inputs(3, 1, h_q, "bf16", seqlens=(300, 129, 64), seed=78, kv_dtype="fp8")
    x.k_scale[int(x.block_table[0, 1])] *= -1.5
    x.k_scale[int(x.block_table[1, 0])] = 0.0
    x.k_scale[int(x.block_table[2, 0])] *= -1.0
    out, lse, _ = run(x, 4)
    ref_o, ref_l = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, False)
    compare(out, lse, ref_o, ref_l, "fp8 negative / zero page scales", tol_o=range_tol(ref_o))


@pytest.mark.parametrize("h_q", [16, 128])
def test_fp8_unused_slots_and_pages_are_never_read_bitwise(h_q):
    _say(f"fp8: NaN codes in unused slots and pages, h_q={h_q}")
    seqlens = (70, 130, 3)
    x = make_inputs(3, 1, h_q, "bf16", seqlens=seqlens, seed=29, extra_pages=4, kv_dtype="fp8")
    out1, lse1, _ = run(x, 4)
    raw = x.k_cache.view(torch.uint8)
    for b, nlen in enumerate(seqlens):
        p = (nlen + 63) // 64
        raw[int(x.block_table[b, p - 1]), nlen % 64:, 0, :] = 0x7F      # NaN: the slots are never read
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(x.k_cache.shape[0]):
        if page not in used:
            raw[page] = 0x7F                                            # NaN codes
            x.k_scale[page] = float("nan")
    out2, lse2, _ = run(x, 4)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


# ------------------------------------------------- fp8 query-key product --
# The query rows are taken into e4m3 with a power-of-two scale per row
# (MLA_KV_FP8_E4M3_QK8); the oracle applies the same quantization
# (quantize_q_rows, pinned on the CPU) and runs the fp64 attention over the
# quantized q and the dequantized cache, so the bar is the one of the other
# paths: the kernel's fp8 products are exact in fp32.
def qk8_reference(x, causal):
    return oracle_decode(quantize_q_rows(x.q), kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, causal)


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("s_q,h_q,seqlens,causal,mode,parts", FP8_EDGE,
                         ids=[f"sq{c[0]}_hq{c[1]}_{'c' if c[3] else 'n'}_{c[4]}_p{c[5]}" for c in FP8_EDGE])
def test_qk8_small_parity(s_q, h_q, seqlens, causal, mode, parts, entry):
    tag = f"fp8 Q.K {entry} s_q={s_q} h_q={h_q} seqlens={seqlens} causal={causal} scale={mode} parts={parts}"
    _say(tag)
    x = make_inputs(len(seqlens), s_q, h_q, "bf16", seqlens=seqlens, causal=causal, seed=sum(seqlens) + 11 * h_q,
                    poison=True, extra_pages=2, kv_dtype="fp8", scale_mode=mode)
    out, lse, _ = run(x, parts, entry, qk_fp8=True)
    ref_o, ref_l = qk8_reference(x, causal)
    compare(out, lse, ref_o, ref_l, tag)


def test_qk8_differs_from_the_bf16_query_product():
    # the fp8 rounding of q is visible: the bf16-q oracle is not what the
    # kernel computes, the quantized-q oracle is
    _say("fp8 Q.K: q rounding visible")
    x = make_inputs(2, 1, 128, "bf16", seqlens=(700, 129), seed=91, kv_dtype="fp8")
    out, lse, _ = run(x, 5, qk_fp8=True)
    ref_o, ref_l = qk8_reference(x, False)
    plain_o, plain_l = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, False)
    compare(out, lse, ref_o, ref_l, "fp8 Q.K")
    assert np.abs(lse - plain_l).max() > 4 * np.abs(lse - ref_l).max()


@pytest.mark.parametrize("h_q", [16, 128])
def test_qk8_negative_zero_and_large_scales(h_q):
    _say(f"fp8 Q.K: page scales, h_q={h_q}")
    x = make_inputs(3, 1, h_q, "bf16", seqlens=(300, 129, 64), seed=92, kv_dtype="fp8")
    x.k_scale[int(x.block_table[0, 1])] *= -1.5
    x.k_scale[int(x.block_table[1, 0])] = 0.0
    x.k_scale[int(x.block_table[2, 0])] *= 3.0
    x.q[0, 0, 0] = 0.0                                   # one all-zero query row
    out, lse, _ = run(x, 4, qk_fp8=True)
    ref_o, ref_l = qk8_reference(x, False)
    compare(out, lse, ref_o, ref_l, "fp8 Q.K page scales", tol_o=range_tol(ref_o))


@pytest.mark.parametrize("h_q", [16, 128])
def test_qk8_unused_slots_and_pages_are_never_read_bitwise(h_q):
    _say(f"fp8 Q.K: NaN codes in unused slots and pages, h_q={h_q}")
    seqlens = (70, 130, 3)
    x = make_inputs(3, 1, h_q, "bf16", seqlens=seqlens, seed=93, extra_pages=4, kv_dtype="fp8")
    out1, lse1, _ = run(x, 4, qk_fp8=True)
    raw = x.k_cache.view(torch.uint8)
    for b, nlen in enumerate(seqlens):
        p = (nlen + 63) // 64
        raw[int(x.block_table[b, p - 1]), nlen % 64:, 0, :] = 0x7F
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(x.k_cache.shape[0]):
        if page not in used:
            raw[page] = 0x7F
            x.k_scale[page] = float("nan")
    out2, lse2, _ = run(x, 4, qk_fp8=True)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("idx", [11, 6])
def test_qk8_full_size_every_request(idx):
    # the headline shape (64-row kernel) and the 128-request varlen shape
    # (16-row kernel) with an fp8 cache and the fp8 query-key product
    w = WORKLOADS[idx]
    _say(f"fp8 Q.K full size: {w.name}")
    host = workload_inputs(idx)
    g = host.to(torch.device("cuda:0"))
    out, lse = api.mla_decode(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, g.causal,
                              k_scale=g.k_scale, qk_fp8=True)
    torch.cuda.synchronize()
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    qd = quantize_q_rows(host.q)
    kv = dequantize_cache(host.k_cache, host.k_scale)
    num = den = 0.0
    for b in range(w.batch):
        o, l = oracle_decode_rows(qd, kv, host.block_table, host.cache_seqlens, host.softmax_scale, host.causal, b)
        o = o.reshape(out[b].shape)
        l = l.reshape(lse[b].shape)
        assert np.abs(out[b] - o).max() <= TOL_O and np.abs(lse[b] - l).max() <= TOL_LSE, f"request {b}"
        num += float(((out[b] - o) ** 2).sum())
        den += float((o ** 2).sum())
    assert math.sqrt(num / den) <= 1e-2


# ------------------------------------------------------------ invariants --
def test_page_permutation_is_bitwise_invariant():
    _say("page permutation invariance")
    x = make_inputs(4, 2, 64, "bf16", seqlens=(300, 64, 129, 1), causal=True, seed=17, extra_pages=2)
    out1, lse1, _ = run(x, 5)
    n = x.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(n)
    x.k_cache = x.k_cache[perm].contiguous()
    used = x.block_table >= 0
    x.block_table[used] = inv[x.block_table[used].long()].to(torch.int32)
    out2, lse2, _ = run(x, 5)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_unused_slots_are_never_read_bitwise():
    _say("garbage in unused slots and pages")
    x = make_inputs(3, 1, 16, "fp16", seqlens=(70, 130, 3), seed=23, poison=True, extra_pages=4)
    out1, lse1, _ = run(x, 4)
    for b, nlen in enumerate((70, 130, 3)):
        p = (nlen + 63) // 64
        x.k_cache[int(x.block_table[b, p - 1]), nlen % 64:, 0, :] = -1000.0
    used = set(int(v) for v in x.block_table.flatten().tolist() if v >= 0)
    for page in range(x.k_cache.shape[0]):
        if page not in used:
            x.k_cache[page] = 777.0
    out2, lse2, _ = run(x, 4)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("s_q,h_q,dtype", [(1, 16, "bf16"), (1, 128, "bf16"), (2, 64, "fp16"), (3, 5, "fp16")])
def test_nan_inf_in_unused_slots_never_reach_the_output(s_q, h_q, dtype, entry):
    """Slots past a request's length in its last page hold NaN and +-Inf (as a
    cache allocated with torch.empty may): the result must equal the one with
    finite garbage there, bit for bit, and match the oracle.  A kernel that
    loads those slots and multiplies them by P = 0 would turn the whole request
    into NaN."""
    seqlens = (70, 130, 3, 64, 200)
    _say(f"NaN/Inf in unused slots {entry} s_q={s_q} h_q={h_q} {dtype}")
    x = make_inputs(len(seqlens), s_q, h_q, dtype, seqlens=seqlens, seed=57 + h_q, poison=True,
                    extra_pages=2, causal=s_q > 1)
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, x.causal)
    out1, lse1, _ = run(x, 3, entry)
    for b, nlen in enumerate(seqlens):
        if nlen % 64:
            pg = int(x.block_table[b, (nlen + 63) // 64 - 1])
            tail = x.k_cache[pg, nlen % 64:, 0, :]
            tail[0::2] = float("nan")
            tail[1::2] = float("inf")
            tail[1::2, 1::2] = float("-inf")
    out2, lse2, _ = run(x, 3, entry)
    assert not np.isnan(out2).any() and not np.isnan(lse2).any()
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
    compare(out2, lse2, ref_o, ref_l, "nan tail")


@pytest.mark.parametrize("h_q", [16, 128])
def test_split_counts_agree(h_q):
    _say(f"one partition vs many partitions h_q={h_q}")
    x = make_inputs(5, 1, h_q, "bf16", seqlens=(900, 33, 2000, 640, 1), seed=31)
    o1, l1, _ = run(x, 1)
    o2, l2, m2 = run(x, 17)
    assert (np.diff(m2[1]) > 1).any(), "expected some split requests"
    assert np.abs(o1 - o2).max() <= 2e-3
    assert np.abs(l1 - l2).max() <= 1e-4


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("h_q,seqlens,parts", [
    (16, (12800, 70), 150),        # ~100 pieces: the combine reduces its LSEs in groups of 64
    (128, (25600, 1, 640), 256),   # ~200 pieces: four groups, the last partial
], ids=["hq16_100pieces", "hq128_200pieces"])
def test_requests_cut_into_more_than_64_pieces(h_q, seqlens, parts, entry):
    _say(f"many pieces {entry} h_q={h_q} seqlens={seqlens} parts={parts}")
    x = make_inputs(len(seqlens), 1, h_q, "bf16", seqlens=seqlens, seed=61 + h_q, poison=True)
    out, lse, meta = run(x, parts, entry)
    pieces = np.diff(meta[1])
    assert pieces.max() > 64, f"expected a request cut into more than 64 pieces, got {pieces.max()}"
    ref_o, ref_l = oracle_decode(x.q, kv64(x), x.block_table, x.cache_seqlens, x.softmax_scale, False)
    compare(out, lse, ref_o, ref_l, f"many pieces h_q={h_q}")


# ------------------------------------------------------------ fused path --
@pytest.mark.parametrize("h_q", [16, 128])
def test_fused_repeated_calls_reuse_counters(h_q):
    """The fused merge's arrival counters live in the workspace: consecutive
    calls with different piece counts on one set of buffers agree with the
    two-kernel path, and leave the counters at zero."""
    dev = torch.device("cuda:0")
    parts = 17
    cases = [(900, 33, 2000, 640, 1), (300, 5000, 64, 64, 2), (1, 2, 3, 4000, 700)]
    bufs = None
    for i, seqlens in enumerate(cases):
        _say(f"fused repeated call {i} h_q={h_q} seqlens={seqlens} parts={parts}")
        x = make_inputs(len(seqlens), 1, h_q, "bf16", seqlens=seqlens, seed=40 + i)
        if bufs is None:
            bufs = api.DecodeBuffers(x.q.to(dev), parts)
        o_ref, l_ref, meta = run(x, parts, "mla_decode")
        assert (np.diff(meta[1]) > 1).any(), "expected split requests"
        o_f, l_f, _ = run(x, parts, "mla_decode_fused", buffers=bufs)
        # the two merges round differently in fp32: at most one bf16 step apart
        assert np.all(np.abs(o_f - o_ref) <= 2.0 ** -7 * np.abs(o_ref) + 1e-6)
        assert np.abs(l_f - l_ref).max() <= 1e-5
        # the counters are the first 256 bytes of this workspace (5 requests)
        assert not bufs.workspace[:256].any(), "arrival counters were not reset"


# ------------------------------------------------------------ full size --
# RMS of the output error relative to the RMS of the output, over a whole
# workload: an alarm beside the absolute bounds, which are loose where |O| is
# small (two-token fp16 decode with sigma 0.5 has |O| of a few 1e-3).
TOL_RMS_REL = 1e-2
_FULL_REF = {}


def _full_reference(idx, x):
    """Oracle output of every request of a full-size workload (computed once
    per module, shared by both entry points)."""
    if idx not in _FULL_REF:
        w = WORKLOADS[idx]
        qf = x.q.double().numpy()
        kf = kv64(x)
        _FULL_REF[idx] = [oracle_decode_rows(qf, kf, x.block_table, x.cache_seqlens, x.softmax_scale, w.causal, b)
                          for b in range(w.batch)]
    return _FULL_REF[idx]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("idx", [2, 3, 4, 5, 6, 11, 12])
def test_workload_full_size_every_request(idx, entry):
    """Full-size workload in the launch configuration the benchmark uses;
    every request is checked against the oracle (max |dO|, max |dLSE|), and
    the RMS-relative output error over the whole workload is bounded."""
    w = WORKLOADS[idx]
    _say(f"workload {idx} {w.name} full size ({entry})")
    x = workload_inputs(idx)
    out, lse, meta = run(x, entry=entry)
    ref = _full_reference(idx, x)
    R = w.s_q * w.h_q
    num = den = 0.0
    for b in range(w.batch):
        ref_o, ref_l = ref[b]
        o = out[b].reshape(R, 512)
        compare(o, lse[b].reshape(R), ref_o, ref_l, f"workload {idx} request {b}")
        num += float(((o - ref_o) ** 2).sum())
        den += float((ref_o ** 2).sum())
    rms_rel = (num / den) ** 0.5
    _say(f"workload {idx} rms_rel_dO = {rms_rel:.3e}")
    assert rms_rel <= TOL_RMS_REL, f"workload {idx}: RMS-relative dO = {rms_rel}"
    assert np.isfinite(lse).all()


# ------------------------------------------------ context-parallel shards --
def _shard(x, r, n_shards):
    """Shard r of every request: pages [r*P//N, (r+1)*P//N) of the request's P
    pages, as a stand-alone batch (same page pool, its own block table and
    lengths)."""
    B = x.block_table.shape[0]
    bt = torch.full_like(x.block_table, -1)
    lens = torch.zeros_like(x.cache_seqlens)
    for b in range(B):
        n = int(x.cache_seqlens[b])
        P = (n + 63) // 64
        lo, hi = r * P // n_shards, (r + 1) * P // n_shards
        if lo < hi:
            bt[b, :hi - lo] = x.block_table[b, lo:hi]
            lens[b] = min(n, hi * 64) - lo * 64
    return bt, lens


@pytest.mark.parametrize("s_q,h_q,n_shards,causal", [(1, 16, 3, False), (1, 128, 4, False),
                                                     (2, 64, 3, True), (1, 16, 8, False)])
def test_context_parallel_shards_merge(s_q, h_q, n_shards, causal):
    """Every shard of the requests runs mla_decode on its own token range (the
    shard holding the last tokens with the causal mask, the others without);
    mla_merge_partials of the shard results equals the whole-request oracle."""
    _say(f"context-parallel merge s_q={s_q} h_q={h_q} shards={n_shards} causal={causal}")
    seqlens = (1000, 3000, 130, 64)          # 64: one page, so some shards are empty
    x = make_inputs(len(seqlens), s_q, h_q, "bf16", seqlens=seqlens, causal=causal, seed=51 + h_q,
                    poison=True)
    dev = torch.device("cuda:0")
    g = x.to(dev)
    outs, lses = [], []
    for r in range(n_shards):
        bt, lens = _shard(x, r, n_shards)
        bt, lens = bt.to(dev), lens.to(dev)
        last = r == n_shards - 1
        o, l = api.mla_decode(g.q, g.k_cache, bt, lens, g.softmax_scale, causal and last)
        outs.append(o.clone())
        lses.append(l.clone())
    part_out = torch.stack(outs)
    part_lse = torch.stack(lses)
    out, lse = api.mla_merge_partials(part_out, part_lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "context-parallel merge")
    whole_o, whole_l, _ = run(x)
    assert np.abs(out.float().cpu().numpy() - whole_o).max() <= 1e-2
    assert np.abs(lse.cpu().numpy() - whole_l).max() <= 1e-4


def test_merge_all_shards_empty():
    """Rows that no shard saw: O = 0, LSE = -inf."""
    _say("merge of shards that saw no key")
    dev = torch.device("cuda:0")
    part_out = torch.randn(3, 2, 1, 16, 512, device=dev).to(torch.bfloat16)
    part_lse = torch.full((3, 2, 1, 16), float("-inf"), device=dev)
    part_lse[1, 1] = 0.5
    out, lse = api.mla_merge_partials(part_out, part_lse)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0]).all() and not out[0].any()
    assert torch.allclose(out[1].float(), part_out[1, 1].float()) and torch.allclose(lse[1], part_lse[1, 1])
