"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds tests/sanitize/host_checks.cpp against an instrumented copy of the
repack code (csrc/pack.cpp) and of the argument validation (csrc/moe_api.hip,
host code only: the sanitizer flags reach the host compilation alone), linked
with the library's other objects as built for gfx950, and runs it: repack round
trips of all three expert formats and every refusal of every entry point.  No
GPU is touched (each refused call returns before any HIP call), so this runs
with the CPU tests.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_routed_expert_moe_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")
# objects of the kernels and launchers, linked uninstrumented
OTHER_OBJECTS = ["route.o", "dispatch.o", "ffn.o", "ffn_decode.o", "ffn_prefill.o", "ffn_prefill_f8.o", "combine.o"]
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _tools():
    hipcc = os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else
                                        shutil.which("hipcc"))
    gxx = shutil.which("g++")
    return hipcc, gxx


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_abi_under_asan_and_ubsan(tmp_path):
    hipcc, gxx = _tools()
    if not hipcc or not gxx:
        pytest.skip("needs hipcc and g++")
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in OTHER_OBJECTS):
        from mxfp4_routed_expert_moe_amd import build as _build
        _build.build()
    out = str(tmp_path)
    api_o = os.path.join(out, "moe_api_san.o")
    # each sanitizer flag applies to the host compilation only
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, "moe_api.hip"),
          "-o", api_o, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san])
    pack_o = os.path.join(out, "pack_san.o")
    _run([gxx, "-O1", "-g", "-std=c++17", "-fPIC", *SAN, "-c", os.path.join(CSRC, "pack.cpp"), "-o", pack_o])
    drv_o = os.path.join(out, "host_checks.o")
    _run([gxx, "-O1", "-g", "-std=c++17", *SAN, "-c", DRIVER, "-o", drv_o])
    exe = os.path.join(out, "host_checks")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    _run([gxx, *SAN, drv_o, api_o, pack_o, *[os.path.join(BUILD, o) for o in OTHER_OBJECTS], "-o", exe,
          f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks passed" in r.stdout, f"rc={r.returncode}\n{r.stdout}\n{r.stderr}"
