"""The boundary's host code (argument checks, status strings, size arithmetic,
codebook validation) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven by a C program through every entry point of include/fq.h, on the CPU
(no GPU call succeeds here, so only the host paths run).  Device code is built
without sanitizers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "universal_vector_quantization_amd", "csrc")
OBJS = os.path.join(ROOT, "_build")
OUT = os.path.join(OBJS, "abi_sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.mark.slow
def test_host_argument_layer_under_asan_and_ubsan():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not installed")
    kernel_objs = sorted(os.path.join(OBJS, f) for f in os.listdir(OBJS) if f.endswith(".o") and f != "fq_api.o") \
        if os.path.isdir(OBJS) else []
    if not kernel_objs:
        pytest.skip("library objects not built (run the library build first)")
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "fq_api_san.o")
    drv_o = os.path.join(OUT, "abi_host_checks.o")
    exe = os.path.join(OUT, "abi_host_checks")
    # host code of the boundary with the sanitizers (each -fsanitize= applies to the host pass only)
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, "fq_api.hip"), "-o", api_o])
    _run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "abi_host", "abi_host_checks.c"),
          "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          drv_o, api_o, *kernel_objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "abi host checks: ok" in r.stdout, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
