"""mla_decode_noalloc: mla_decode with the workspace in the library's static
per-GPU array, called through the C ABI.  Two calls in a row (the second on a
smaller input, so the array holds the first call's leftovers) must equal
mla_decode on the same inputs and match the oracle within the usual
tolerances; a shape whose workspace exceeds the array is refused on the host."""

import sys

import numpy as np
import pytest
import torch

from oracle import oracle_decode
from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

TOL_O = 1.5e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    yield
    torch.cuda.synchronize()


CASES = [
    # (s_q, h_q, seqlens, causal, dtype, num_parts): larger first, then smaller
    (1, 128, (3000, 70, 1, 2100, 640, 129), False, "bf16", 17),
    (2, 16, (700, 1, 265), True, "fp16", 7),
]


def test_noalloc_equals_mla_decode_on_two_calls():
    dev = torch.device("cuda:0")
    for i, (s_q, h_q, seqlens, causal, dtype, parts) in enumerate(CASES):
        print(f"noalloc call {i}: s_q={s_q} h_q={h_q} seqlens={seqlens} {dtype} parts={parts}", flush=True)
        sys.stdout.flush()
        x = make_inputs(len(seqlens), s_q, h_q, dtype, seqlens=seqlens, causal=causal, seed=90 + i,
                        poison=True, extra_pages=2)
        g = x.to(dev)
        meta = api.get_metadata(g.cache_seqlens, s_q, h_q, num_parts=parts)
        assert (np.diff(meta[1].cpu().numpy()) > 1).any(), "expected split requests"
        ref_out, ref_lse = api.mla_decode(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, causal,
                                          metadata=meta)
        out, lse = api.mla_decode_noalloc(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, causal,
                                          metadata=meta)
        torch.cuda.synchronize()
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        assert np.array_equal(o, ref_out.float().cpu().numpy()) and np.array_equal(l, ref_lse.cpu().numpy())
        ref_o, ref_l = oracle_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, causal)
        fin = np.isfinite(ref_l)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.abs(o - ref_o).max() <= TOL_O
        assert np.abs(l[fin] - ref_l[fin]).max() <= TOL_LSE


def test_noalloc_refuses_a_workspace_beyond_the_static_array():
    dev = torch.device("cuda:0")
    print("noalloc: workspace beyond the static array", flush=True)
    x = make_inputs(64, 1, 128, "bf16", seqlens=(1,) * 64, seed=7)
    g = x.to(dev)
    parts = 256          # (64 + 256) pieces x 128 rows x 513 x 4 bytes > 64 MiB
    meta = api.get_metadata(g.cache_seqlens, 1, 128, num_parts=parts)
    assert api.workspace_size(64, 1, 128, parts) > 64 << 20
    with pytest.raises(api.MlaError) as err:
        api.mla_decode_noalloc(g.q, g.k_cache, g.block_table, g.cache_seqlens, g.softmax_scale, False,
                               metadata=meta)
    assert err.value.status == 3 and "static workspace" in str(err.value)
