"""Host-side checks of bench.py: the algorithmic byte and FLOP counts behind
its roofline figures, re-derived here from the definition (2 h_q s_q s_k
(576 + 512) FLOP per request; the cached rows once, V inside K) on the seeded
workloads; the kernel each workload is attributed to; the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_decode_attention_02_amd.workloads import MHA_WORKLOADS, WORKLOADS, workload_seqlens  # noqa: E402


def _mla_counts(idx):
    w = WORKLOADS[idx]
    sl = workload_seqlens(idx)
    return w, sl, bench.algorithmic_counts(sl, w.batch, w.s_q, w.h_q, kv_elem=1 if w.kv == "fp8" else 2)


# (workload, KV MB, algorithmic bytes MB, GFLOP), to 0.01: the measurement
# table of the configurations (KV once, + Q, O, LSE and the table entries read)
TABLE = [(2, 301.99, 319.87, 73.01), (3, 632.17, 636.67, 19.11), (4, 528.67, 546.55, 255.64),
         (5, 490.73, 491.88, 118.65)]


@pytest.mark.parametrize("idx,kv_mb,bytes_mb,gflop", TABLE)
def test_mla_counts_match_the_configuration_table(idx, kv_mb, bytes_mb, gflop):
    w, sl, (flops, kv, q, o, lse, tb) = _mla_counts(idx)
    assert round(kv / 1e6, 2) == kv_mb
    assert round((kv + q + o + lse + tb) / 1e6, 2) == bytes_mb
    assert round(flops / 1e9, 2) == gflop


def test_mla_counts_by_hand_on_the_headline_workload():
    w, sl, (flops, kv, q, o, lse, tb) = _mla_counts(2)
    assert sl == [4096] * 64
    assert flops == 2 * 128 * 4096 * (576 + 512) * 64
    assert kv == 64 * 4096 * 576 * 2
    assert q == 64 * 128 * 576 * 2 and o == 64 * 128 * 512 * 2 and lse == 64 * 128 * 4
    assert tb == 64 * 64 * 4 + 64 * 4


def test_fp8_counts_halve_the_cache_and_add_the_scales():
    sl = workload_seqlens(6)
    f2, kv2, *_ = bench.algorithmic_counts(sl, 128, 1, 16, kv_elem=2)
    f1, kv1, *_ = bench.algorithmic_counts(sl, 128, 1, 16, kv_elem=1)
    pages = sum((n + 63) // 64 for n in sl)
    assert f1 == f2 and kv1 == kv2 // 2 + 4 * pages


def test_mha_counts():
    w = MHA_WORKLOADS[7]
    sl = workload_seqlens(7)
    flops, kv, q, o, lse, tb = bench.mha_algorithmic_counts(sl, w.batch, w.s_q, w.h_q, w.h_kv, w.head_dim)
    assert flops == sum(2 * 64 * n * 256 for n in sl)
    assert kv == sum(sl) * 8 * 128 * 2 * 2
    pages = sum((n + 63) // 64 for n in sl)
    _, kv8, *_ = bench.mha_algorithmic_counts(sl, w.batch, w.s_q, w.h_q, w.h_kv, w.head_dim, kv_elem=1)
    assert kv8 == kv // 2 + pages * 8 * 2 * 4


def test_kernel_attribution():
    # the split-KV kernel each workload runs, as the library dispatches it
    # (16 rows or fewer: narrow; more: wide; fp8 cache: the fp8 kernel of the
    # same width; MHA: key split for fp8 caches with small row tiles, else
    # mha_splitkv_kernel)
    assert [bench.mla_kernel_name(WORKLOADS[i]) for i in (13, 14, 15)] == ["splitkv_wide_fp8_kernel"] * 2 + [
        "splitkv_fp8_kernel"]
    assert [bench.mla_kernel_name(WORKLOADS[i]) for i in (1, 2, 3, 4, 5, 6, 11, 12)] == [
        "splitkv_narrow_kernel", "splitkv_wide_kernel", "splitkv_narrow_kernel", "splitkv_wide_kernel",
        "splitkv_wide_kernel", "splitkv_fp8_kernel", "splitkv_wide_fp8_kernel", "splitkv_wide_fp8_kernel"]
    assert [bench.mha_kernel_name(MHA_WORKLOADS[i]) for i in (7, 8, 9, 10)] == [
        "mha_splitkv_kernel", "mha_splitkv_kernel", "mha_keysplit_kernel", "mha_splitkv_kernel"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_mla_record_rates_use_the_timed_step_count():
    # the region is divided by the steps timed, not by the number of steps
    # that carried timing events (one in EVENT_STRIDE)
    import types

    import torch

    from mla_decode_attention_02_amd.workloads import WORKLOADS, workload_seqlens

    w = WORKLOADS[2]
    steps = 200
    sampled = steps // bench.EVENT_STRIDE
    m = {"workload": w, "host": types.SimpleNamespace(cache_seqlens=torch.tensor(workload_seqlens(2))),
         "num_parts": 128, "fixed_overhead": 2, "copies": 2, "steps": steps,
         "region_ms": steps * 0.1, "step_ms": [0.099] * sampled, "splitkv_ms": [0.09] * sampled,
         "combine_ms": [0.009] * sampled, "meta_ms": None, "pre_step_ms": None, "pre_splitkv_ms": None}
    rec = bench.mla_record(2, m, {"step_ms": [0.098] * 5})
    assert rec["ms_per_step_region"] == 0.1
    flops = bench.algorithmic_counts(workload_seqlens(2), w.batch, w.s_q, w.h_q)[0]
    assert abs(rec["step_tflops"] - flops / 1e-4 / 1e12) < 0.01
    assert rec["splitkv_us"]["median"] == 90.0 and rec["metadata_us_median"] is None


def test_fp8_query_key_path_is_priced_at_the_blended_mfma_peak():
    # Q.K^T (576 of 1088 FLOPs per row and key) at the fp8 rate, P.V at the
    # bf16 rate: the time at peak is the sum of the two shares' times
    assert bench.mla_mfma_peak(False) == bench.MFMA_PEAK_TFLOPS
    peak = bench.mla_mfma_peak(True)
    assert abs(peak - 3400.0) < 1e-9
    t = 576 / bench.MFMA_FP8_PEAK_TFLOPS + 512 / bench.MFMA_PEAK_TFLOPS
    assert abs(1088 / t - peak) < 1e-9
    assert bench.MFMA_PEAK_TFLOPS < peak < bench.MFMA_FP8_PEAK_TFLOPS
