"""The decode paths under HIP graph capture: the schedule, the split-KV kernel
and the combine are recorded once on torch's capture stream and replayed; every
replay (with eager work and synchronisations in between) must equal the eager
result bit for bit, for the two-kernel MLA path, the fused path (whose arrival
counters must come back to zero inside the graph) and the MHA path."""

import sys

import pytest
import torch

from mla_decode_attention_02_amd import api
from mla_decode_attention_02_amd.workloads import make_inputs, make_mha_inputs

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


def _replays_match(run, eager_out, n=3):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                   # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        outs = run()
    for i in range(n):
        # eager work between replays, then the replay
        junk = torch.randn(1 << 20, device="cuda:0").sum()
        torch.cuda.synchronize()
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager_out):
            assert torch.equal(a, b), f"replay {i} differs from the eager result"
        del junk


@pytest.mark.parametrize("entry", ["mla_decode", "mla_decode_fused"])
@pytest.mark.parametrize("h_q", [16, 128])
def test_mla_graph_replay(entry, h_q):
    _say(f"graph replay {entry} h_q={h_q}")
    x = make_inputs(4, 1, h_q, "bf16", seqlens=(900, 33, 2000, 1), seed=61).to(torch.device("cuda:0"))
    parts = 17
    meta = api.get_metadata(x.cache_seqlens, 1, h_q, num_parts=parts)
    bufs = api.DecodeBuffers(x.q, parts)
    fn = getattr(api, entry)
    o, l = fn(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False, metadata=meta, buffers=bufs)
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.DecodeBuffers(x.q, parts)

    def run():
        m = api.get_metadata(x.cache_seqlens, 1, h_q, num_parts=parts)
        return fn(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False, metadata=m, buffers=gbufs)

    _replays_match(run, eager)
    if entry == "mla_decode_fused":
        assert not gbufs.workspace[:256].any(), "arrival counters not reset inside the graph"


def test_fp8_graph_replay():
    _say("graph replay fp8 cache")
    x = make_inputs(3, 1, 16, "bf16", seqlens=(700, 64, 5), seed=62, kv_dtype="fp8").to(torch.device("cuda:0"))
    meta = api.get_metadata(x.cache_seqlens, 1, 16, num_parts=9)
    o, l = api.mla_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False,
                          metadata=meta, k_scale=x.k_scale)
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.DecodeBuffers(x.q, 9)

    def run():
        m = api.get_metadata(x.cache_seqlens, 1, 16, num_parts=9)
        return api.mla_decode(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False,
                              metadata=m, buffers=gbufs, k_scale=x.k_scale)

    _replays_match(run, eager)


def test_mha_graph_replay():
    _say("graph replay MHA")
    x = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(1500, 64, 7), seed=63).to(torch.device("cuda:0"))
    meta = api.mha_get_metadata(x.cache_seqlens, 1, 16, 4, num_parts=11)
    o, l = api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=meta)
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.MhaBuffers(x.q, 4, 11)

    def run():
        m = api.mha_get_metadata(x.cache_seqlens, 1, 16, 4, num_parts=11)
        return api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=m, buffers=gbufs)

    _replays_match(run, eager)


def test_mha_fp8_graph_replay():
    _say("graph replay MHA, fp8 K/V caches")
    x = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(1500, 64, 7), seed=64,
                        kv_dtype="fp8").to(torch.device("cuda:0"))
    meta = api.mha_get_metadata(x.cache_seqlens, 1, 16, 4, num_parts=11)
    o, l = api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=meta,
                          k_scale=x.k_scale, v_scale=x.v_scale)
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.MhaBuffers(x.q, 4, 11)

    def run():
        m = api.mha_get_metadata(x.cache_seqlens, 1, 16, 4, num_parts=11)
        return api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=m, buffers=gbufs,
                              k_scale=x.k_scale, v_scale=x.v_scale)

    _replays_match(run, eager)


@pytest.mark.parametrize("entry", ["mla_decode", "mla_decode_fused"])
@pytest.mark.parametrize("h_q,kv", [(16, "same"), (128, "same"), (16, "fp8")])
def test_mla_graph_replay_schedule_in_kernels(entry, h_q, kv):
    # no schedule passed: the graph holds only the split-KV kernel and the
    # combine, both deriving the schedule from cache_seqlens on every replay
    _say(f"graph replay {entry} h_q={h_q} kv={kv}, schedule in the kernels")
    x = make_inputs(4, 1, h_q, "bf16", seqlens=(900, 33, 2000, 1), seed=65, kv_dtype=kv).to(torch.device("cuda:0"))
    parts = 17
    fn = getattr(api, entry)
    o, l = fn(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False, metadata=parts,
              buffers=api.DecodeBuffers(x.q, parts), k_scale=x.k_scale)
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.DecodeBuffers(x.q, parts)

    def run():
        return fn(x.q, x.k_cache, x.block_table, x.cache_seqlens, x.softmax_scale, False, metadata=parts,
                  buffers=gbufs, k_scale=x.k_scale)

    _replays_match(run, eager)


def test_mha_graph_replay_schedule_in_kernels():
    _say("graph replay MHA, schedule in the kernels")
    x = make_mha_inputs(3, 1, 16, 4, 128, "bf16", seqlens=(1500, 64, 7), seed=66).to(torch.device("cuda:0"))
    o, l = api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=11,
                          buffers=api.MhaBuffers(x.q, 4, 11))
    torch.cuda.synchronize()
    eager = (o.clone(), l.clone())
    gbufs = api.MhaBuffers(x.q, 4, 11)

    def run():
        return api.mha_decode(x.q, x.k_cache, x.v_cache, x.block_table, x.cache_seqlens, metadata=11,
                              buffers=gbufs)

    _replays_match(run, eager)
