"""The C ABI's host code (argument validation, status and error strings,
workspace sizing) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven by tests/host/validation_main.cpp.  The sanitizers instrument the
host code only (each -fsanitize flag follows -Xarch_host); every call the
driver makes fails validation before any HIP call, except one failed launch
when no HIP device is visible."""

import os
import shutil
import subprocess

import pytest

from kv_cache_calibration_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_sanitize")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.slow
def test_validation_under_host_asan_and_ubsan():
    if not (shutil.which(B.HIPCC) or os.path.exists(B.HIPCC)) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang++ not available")
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        extra = SAN if src == "nsn_api.hip" else []
        _run([B.HIPCC, *B.FLAGS, *extra, "-c", os.path.join(B.CSRC, src), "-o", obj])
        objs.append(obj)
    # the driver is plain C++ (it includes only nsn.h): compile and link it
    # with the host clang, against the HIP runtime
    exe = os.path.join(OUT, "validation")
    main_o = os.path.join(OUT, "validation_main.o")
    _run([CLANG, "-O1", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "host", "validation_main.cpp"), "-o", main_o])
    _run([CLANG, "-fsanitize=address,undefined", main_o, *objs, "-L", ROCM_LIB,
          "-Wl,-rpath," + ROCM_LIB, "-lamdhip64", "-o", exe])
    try:
        import torch
        no_device = torch.cuda.device_count() == 0
    except ImportError:
        no_device = False
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the life of the process
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [exe] + (["--no-device"] if no_device else [])
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{r.stdout}\n{r.stderr}"
    assert "ok: 0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
