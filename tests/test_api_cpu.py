"""The binding fails loudly, before any compute, on inputs the library cannot
take: host tensors, mismatched dtypes or shapes.  There is no CPU fallback."""

import pytest
import torch

from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import make_inputs, make_mha_inputs


def test_mla_rejects_host_tensors():
    x = make_inputs(2, 1, 16, "bf16", seqlens=(64, 3), seed=1)
    with pytest.raises(ValueError):
        api.mla_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False,
                       metadata=(torch.zeros(4, 8, dtype=torch.int32), torch.zeros(3, dtype=torch.int32)))


def test_mla_rejects_dtype_mismatch():
    x = make_inputs(2, 1, 16, "bf16", seqlens=(64, 3), seed=1)
    with pytest.raises(ValueError):
        api._validate_tensors(x.q, x.k_cache.half(), x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):
        api._validate_tensors(x.q.half(), x.k_cache.to(torch.float8_e4m3fn), x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):                    # a scale array needs an fp8 cache
        api._validate_tensors(x.q, x.k_cache, x.block_table, x.cache_seqlens,
                              k_scale=torch.ones(x.k_cache.shape[0]))


def test_mha_rejects_mismatches():
    x = make_mha_inputs(2, 1, 8, 2, 64, "bf16", seqlens=(64, 3), seed=1)
    with pytest.raises(ValueError):
        api._validate_mha(x.q, x.k_cache, x.v_cache.half(), x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):
        api._validate_mha(x.q, x.k_cache, x.v_cache[..., :32], x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):                    # host tensors
        api._validate_mha(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens)


def test_metadata_needs_device_lengths():
    with pytest.raises(ValueError):
        api.get_metadata(torch.tensor([3, 4], dtype=torch.int32), 1, 16)
    with pytest.raises(ValueError):
        api.mha_get_metadata(torch.tensor([3, 4], dtype=torch.int32), 1, 8, 2)


def test_mha_fp8_rejects_mismatches():
    x = make_mha_inputs(2, 1, 8, 2, 64, "bf16", seqlens=(64, 3), seed=1, kv_dtype="fp8")
    n, h = x.k_cache.shape[0], x.k_cache.shape[2]
    with pytest.raises(ValueError):                    # fp8 K with a bf16 V
        api._validate_mha(x.q, x.k_cache, x.v_cache.to(torch.bfloat16), x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):                    # fp8 caches need a bf16 q
        api._validate_mha(x.q.half(), x.k_cache, x.v_cache, x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):                    # one scale per page and KV head
        api._validate_mha(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, k_scale=torch.ones(n))
    with pytest.raises(ValueError):
        api._validate_mha(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens,
                          v_scale=torch.ones(n, h, dtype=torch.float64))
    y = make_mha_inputs(2, 1, 8, 2, 64, "bf16", seqlens=(64, 3), seed=1)
    with pytest.raises(ValueError):                    # scales apply to fp8 caches only
        api._validate_mha(y.q, y.k_cache, y.v_cache, y.block_table, y.cache_seqlens, k_scale=torch.ones(n, h))


def test_batch_mismatch_is_rejected():
    """block_table rows, cache_seqlens and q must describe the same requests:
    the schedule is built from the lengths and the kernels index the table by
    request, so a mismatch would read past either array on the device."""
    x = make_inputs(3, 1, 16, "bf16", seqlens=(64, 3, 9), seed=1)
    api._check_batch(x.q, x.block_table, x.cache_seqlens)
    with pytest.raises(ValueError):
        api._check_batch(x.q, x.block_table[:2], x.cache_seqlens)
    with pytest.raises(ValueError):
        api._check_batch(x.q, x.block_table, x.cache_seqlens[:2])
    with pytest.raises(ValueError):
        api._check_batch(x.q[:2], x.block_table, x.cache_seqlens)
    y = make_mha_inputs(3, 1, 8, 2, 64, "bf16", seqlens=(64, 3, 9), seed=1)
    with pytest.raises(ValueError):
        api._check_batch(y.q, y.block_table, y.cache_seqlens[1:])


def test_caller_buffers_are_checked_against_q():
    x = make_inputs(2, 2, 16, "fp16", seqlens=(64, 3), seed=1)
    B, s_q, h_q = 2, 2, 16
    out = torch.empty(B, s_q, h_q, 512, dtype=torch.float16)
    lse = torch.empty(B, s_q, h_q, dtype=torch.float32)
    api._check_outputs(x.q, out, lse, 512)
    api._check_outputs(x.q, torch.empty(B, s_q, h_q, 520, dtype=torch.float16)[..., :512], lse, 512)
    bad = [
        (torch.empty(B, s_q, h_q + 1, 512, dtype=torch.float16), lse),     # wrong heads
        (torch.empty(B, s_q, h_q, 512, dtype=torch.bfloat16), lse),        # wrong dtype
        (torch.empty(B, s_q, h_q, 256, dtype=torch.float16), lse),         # wrong width
        (torch.empty(B, s_q, h_q, 1024, dtype=torch.float16)[..., ::2], lse),  # strided columns
        (out, torch.empty(B, s_q, h_q + 1, dtype=torch.float32)),           # lse shape
        (out, torch.empty(B, s_q, h_q, dtype=torch.float64)),               # lse dtype
        (out, torch.empty(B, h_q, s_q, dtype=torch.float32).transpose(1, 2)),  # lse not contiguous
    ]
    for o, l in bad:
        with pytest.raises(ValueError):
            api._check_outputs(x.q, o, l, 512)


def test_metadata_shape_is_checked():
    dev = torch.device("cpu")
    api._check_metadata(torch.zeros(4, 8, dtype=torch.int32), torch.zeros(6, dtype=torch.int32), 5, dev)
    with pytest.raises(ValueError):       # split_offsets of another batch
        api._check_metadata(torch.zeros(4, 8, dtype=torch.int32), torch.zeros(5, dtype=torch.int32), 5, dev)
    with pytest.raises(ValueError):       # schedule rows of the wrong width
        api._check_metadata(torch.zeros(4, 7, dtype=torch.int32), torch.zeros(6, dtype=torch.int32), 5, dev)
    with pytest.raises(ValueError):       # wrong dtype
        api._check_metadata(torch.zeros(4, 8, dtype=torch.int64), torch.zeros(6, dtype=torch.int32), 5, dev)
