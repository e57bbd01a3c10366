"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tq_host.cpp (argument checks, table builders, calibration, the C entry
points) is compiled for the host only with g++ and both sanitizers, linked
with the HIP objects of the normal build (not instrumented) and driven by
tests/host_sanitize/driver.cpp through every path that needs no GPU.  Any
sanitizer report aborts the driver (-fno-sanitize-recover), so the test
fails on the first one.  No GPU is used: nothing here launches a kernel."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_vector_05_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIP_OBJS = ["tq_gemm.o", "tq_encode.o", "tq_attn.o", "tq_qprep.o", "tq_scan.o", "tq_decode.o", "tq_vq.o",
            "tq_noalloc.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    objs = [os.path.join(BUILD, o) for o in HIP_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (python -m kv_cache_vector_05_amd.build)")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include"]
    host_o, drv_o, exe = (str(tmp_path / n) for n in ("tq_host.o", "driver.o", "driver"))
    _run([gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-ffp-contract=off"] + SAN + inc +
         ["-c", os.path.join(CSRC, "tq_host.cpp"), "-o", host_o])
    _run([gxx, "-std=c++17", "-O1", "-g"] + SAN + inc +
         ["-c", os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"), "-o", drv_o])
    _run([gxx] + SAN + [drv_o, host_o] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = _run([exe], env=env, timeout=300)
    assert "host sanitizer driver: ok" in r.stdout
