"""Pins for the split-KV schedule re-derivation (no GPU).

Hand-derived schedules (tests/golden/metadata_hand_cases.json) fix the exact
format and cutting rule; the invariants below must hold for any input: every
page of every request is covered exactly once, in order, by contiguous chunks;
no partition exceeds the quota ceil(T / parts) + F; partitions hold consecutive
stretches of the request order; split counts and offsets agree with the chunks.
"""

import json
import os
import random

import numpy as np
import pytest

from oracle.metadata import FIXED_OVERHEAD, oracle_metadata, schedule_chunks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE = 64


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "metadata_hand_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_derived_schedules(case):
    sched, offs = oracle_metadata(case["seqlens"], case["num_parts"], case["fixed_overhead"])
    assert sched.tolist() == case["sched"]
    assert offs.tolist() == case["split_offsets"]


def _check_invariants(seqlens, num_parts, F=FIXED_OVERHEAD):
    P = [(n + PAGE - 1) // PAGE for n in seqlens]
    total = sum(p + F for p in P if p > 0)
    quota = -(-total // num_parts) + F
    chunks = schedule_chunks(seqlens, num_parts, F)
    # coverage: per request, chunks are contiguous, ordered, and cover [0, P_b)
    per_req = {}
    for part, b, lo, hi in chunks:
        assert 0 <= lo < hi <= P[b]
        per_req.setdefault(b, []).append((part, lo, hi))
    for b, p in enumerate(P):
        lst = sorted(per_req.get(b, []), key=lambda t: t[1])
        if p == 0:
            assert lst == []
            continue
        assert lst[0][1] == 0 and lst[-1][2] == p
        for (pa, _, h0), (pb, l1, _) in zip(lst, lst[1:]):
            assert h0 == l1 and pb > pa
    # parts hold consecutive stretches of the request order, each within quota
    order = [(c[0], c[1], c[2]) for c in chunks]
    assert order == sorted(order) and all(0 <= c[0] < num_parts for c in chunks)
    flat = sorted(chunks, key=lambda c: (c[1], c[2]))
    assert [c[0] for c in flat] == sorted(c[0] for c in flat)
    spent = {}
    for part, b, lo, hi in chunks:
        spent[part] = spent.get(part, 0) + (hi - lo) + F
    assert all(v <= quota for v in spent.values())
    # sched / offsets agree with the chunks
    sched, offs = oracle_metadata(seqlens, num_parts, F)
    n_splits = [len(per_req.get(b, [])) for b in range(len(P))]
    assert offs[0] == 0 and np.all(np.diff(offs) >= 0)
    assert np.diff(offs).tolist() == n_splits
    assert offs[-1] == len(chunks)
    for part in range(num_parts):
        mine = [c for c in chunks if c[0] == part]
        row = sched[part].tolist()
        if not mine:
            assert row == [0, 0, -1, 0, 0, 0, 0, 0]
            continue
        assert row[0] == mine[0][1] and row[1] == mine[0][2]
        assert row[2] == mine[-1][1] and row[3] == mine[-1][3]
        assert row[5:] == [0, 0, 0]
        # begin_split = index of the first chunk among its request's chunks
        req_chunks = sorted([c for c in chunks if c[1] == mine[0][1]], key=lambda c: c[2])
        assert row[4] == req_chunks.index(mine[0])
        # everything strictly between the first and last request is whole
        for c in mine[1:-1]:
            assert c[2] == 0 and c[3] == P[c[1]]


def _brute_schedule(seqlens, num_parts, F):
    """Unit-by-unit walk of the cost line (independent of the page formula)."""
    P = [(n + PAGE - 1) // PAGE for n in seqlens]
    units = []
    for b, p in enumerate(P):
        if p:
            units += [None] * (F // 2) + [(b, i) for i in range(p)] + [None] * (F - F // 2)
    width = max(1, -(-len(units) // num_parts))
    owner = {}
    for pos, u in enumerate(units):
        if u is not None:
            owner[u] = pos // width
    return owner


@pytest.mark.parametrize("seed", range(12))
def test_matches_unit_walk(seed):
    rng = random.Random(100 + seed)
    B = rng.choice([1, 2, 5, 17])
    seqlens = [rng.choice([0, 1, 63, 64, 65, 200, 700]) for _ in range(B)]
    parts = rng.choice([1, 2, 3, 7, 16])
    owner = _brute_schedule(seqlens, parts, FIXED_OVERHEAD)
    for part, b, lo, hi in schedule_chunks(seqlens, parts):
        for p in range(lo, hi):
            assert owner[(b, p)] == part


@pytest.mark.parametrize("seed", range(40))
def test_random_schedules_hold_invariants(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 2, 3, 7, 64, 128, 300])
    kind = rng.choice(["uniform", "edges", "skew", "zeros"])
    if kind == "uniform":
        seqlens = [rng.randint(1, 8192) for _ in range(B)]
    elif kind == "edges":
        seqlens = [rng.choice([0, 1, 63, 64, 65, 127, 128, 129]) for _ in range(B)]
    elif kind == "skew":
        seqlens = [rng.choice([1, 2, 3]) for _ in range(B)]
        seqlens[rng.randrange(B)] = rng.randint(100000, 140000)
    else:
        seqlens = [0] * B
        seqlens[rng.randrange(B)] = rng.randint(1, 5000)
    num_parts = rng.choice([1, 2, 3, 8, 64, 128, 256])
    _check_invariants(seqlens, num_parts)


def test_all_empty_batch():
    sched, offs = oracle_metadata([0, 0, 0], 4)
    assert schedule_chunks([0, 0, 0], 4) == []
    assert offs.tolist() == [0, 0, 0, 0]
    assert all(row == [0, 0, -1, 0, 0, 0, 0, 0] for row in sched.tolist())


def test_workload_schedules_hold_invariants():
    from mla_decode_attention_02_amd.workloads import workload_seqlens

    for idx, parts in ((1, 256), (2, 128), (3, 256), (4, 64), (5, 128)):
        _check_invariants(workload_seqlens(idx), parts)
