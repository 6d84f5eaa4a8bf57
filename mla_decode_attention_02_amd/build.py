"""Build libmla_decode.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m mla_decode_attention_02_amd.build [-v]

Objects go to _build/ at the repository root; the shared library is written
next to this file.  Every call recompiles.  The compiler's per-kernel resource
report (registers, scratch, occupancy, LDS) is kept in
_build/kernel_resources.json; the CPU tests check from it that no kernel
spills registers or uses scratch memory.
"""

from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_decode.so")
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
SOURCES = ["mla_api.cpp", "mha_api.cpp", "mla_metadata.hip", "mla_splitkv_wide.hip", "mla_splitkv_narrow.hip",
           "mla_splitkv_fp8.hip", "mla_combine.hip", "mla_merge.hip", "mha_decode.hip", "mla_check.hip",
           "mla_splitkv_wide8.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# Per-source extra flags.  The narrow kernel keeps its MFMA accumulators in the
# VGPR form (its per-wave output rescale then needs no AGPR round trips); the
# wide kernel runs faster with the default AGPR form (measured on MI355X).
EXTRA_FLAGS = {"mla_splitkv_narrow.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


_REMARK = "-Rpass-analysis=kernel-resource-usage"


def _resources(stderr: str) -> dict:
    """Per-kernel figures of the compiler's resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?)(?: \[[^\]]*\])?: (\S+) \[" + re.escape(_REMARK), line)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1)] = int(v) if v.lstrip("-").isdigit() else v
    return out


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), _REMARK, "-I", INCLUDE, "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", _REMARK)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj, _resources(res.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in done]
    resources = {src: r for src, (_, r) in zip(SOURCES, done)}
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
