"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the C ABI.

The ABI's host code (argument checks, dispatch, error text, the static
workspace and the device-check plumbing) is built with the sanitizers on the
host side only, linked against stand-ins for the kernel launchers
(tests/sanitize/stub_launchers.hip) and driven by tests/sanitize/abi_driver.cpp
through every entry point's rejections and dispatch, and from eight threads at
once.  No GPU is used; any memory error, leak or undefined behaviour aborts the
driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_decode_attention_02_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
SOURCES = [os.path.join(CSRC, "mla_api.cpp"), os.path.join(CSRC, "mha_api.cpp"), os.path.join(CSRC, "mla_check.hip"),
           os.path.join(SAN, "stub_launchers.hip"), os.path.join(SAN, "abi_driver.cpp")]
# the sanitizers apply to the host side only (each flag after -Xarch_host)
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    flags = ["-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *flags, *HOST_SANITIZE, "-c", src, "-o", obj], capture_output=True, text=True,
                           timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", *objs, "-o", exe, "-lpthread"], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env.pop("MLA_DEBUG", None)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""       # never touch a GPU, even where one exists
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all expectations met" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
