"""The compiled kernels' resource use, from the compiler's report that the
build keeps (_build/kernel_resources.json): no kernel may use scratch memory or
spill registers.  A kernel with a private segment pays scratch set-up on every
launch, and a spill puts memory round trips into its loops; both have crept in
unnoticed from harmless-looking source changes.  Rebuilds first when the report
is missing or older than a source file (CPU only: hipcc cross-compiles)."""

import glob
import json
import os

import pytest

from mla_decode_attention_02_amd import build as B


@pytest.fixture(scope="module")
def resources():
    sources = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(B.INCLUDE, "*"))
    newest = max(os.path.getmtime(p) for p in sources)
    if not os.path.exists(B.RESOURCES) or os.path.getmtime(B.RESOURCES) < newest:
        B.build()
    with open(B.RESOURCES) as f:
        return json.load(f)


def _kernels(res):
    return [(src, name, r) for src, ks in res.items() for name, r in ks.items()]


def test_every_source_reports_its_kernels(resources):
    for src in B.SOURCES:
        if src.endswith(".hip"):
            assert resources.get(src), f"{src}: no kernel in the compiler's report"


def test_no_kernel_uses_scratch_or_spills(resources):
    bad = [(src, name, r.get("ScratchSize"), r.get("VGPRs Spill"))
           for src, name, r in _kernels(resources)
           if r.get("ScratchSize") != 0 or r.get("VGPRs Spill") != 0]
    assert not bad, f"kernels with scratch or VGPR spills: {bad}"


def test_whole_row_combine_keeps_eight_waves_per_simd(resources):
    # the whole-row combine is sized to fit 64 registers (8 waves per SIMD)
    occ = [r["Occupancy"] for name, r in resources["mla_combine.hip"].items() if "Li2E" in name]
    assert occ and all(o == 8 for o in occ), occ
