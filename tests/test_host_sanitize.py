"""The library's host code under the address and undefined-behaviour sanitizers.

api.hip (validation, geometry, workspace sizes, dispatch) is compiled with
-fsanitize=address,undefined on its host side only (the device code is untouched) and
linked with the library's other objects and tests/abi_host_check.cpp, a driver that
walks mbq_describe over a grid of valid and invalid shapes, queries every workspace size
and makes every compute call in forms the library must refuse.  The program runs with
no GPU visible; a sanitizer report or a failed expectation fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def checker():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from token_adaptive_bit_amd import build as B
    objs = [os.path.join(B.BUILD_DIR, s.replace(".hip", ".o")) for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    os.makedirs(OUT, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = os.path.join(OUT, "api.o")
    drv_o = os.path.join(OUT, "abi_host_check.o")
    exe = os.path.join(OUT, "abi_host_check")
    steps = [
        # the library's host code: sanitizers on the host side of the hipcc compile only
        [hipcc, *B.COMMON, "-O1", "-g", *san, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_o],
        # the test program is plain host C++
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
         "-c", os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", drv_o],
        [hipcc, "--offload-arch=gfx950", *san, drv_o, api_o, *objs, "-o", exe],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
    return exe


def test_abi_host_code_is_sanitizer_clean(checker):
    env = dict(os.environ)
    env.update({"HIP_VISIBLE_DEVICES": "-1",
                "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    res = subprocess.run([checker], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, (res.stdout + res.stderr)[-4000:]
    assert "abi host checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
