"""Build libfq.so (the FibQuant HIP library) in-tree for gfx950.

Every kernel source is compiled once per block size k (``-DFQ_ONLY_K=k``) plus
once for its dispatcher, in parallel, then linked into
``universal_vector_quantization_amd/libfq.so``.  Objects go to ``_build/`` at
the repository root.

    python -m universal_vector_quantization_amd.build_lib [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfq.so")
BUILD = os.path.join(ROOT, "_build")
KS = (1, 2, 4, 8, 16, 32, 64)
PER_K = ("fq_encode", "fq_decode", "fq_attn")
# Kernel translation units: no NaN semantics (inputs are finite by contract) so
# min / max need no canonicalisation, and matrix-core results stay in VGPRs.
KERNEL_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_KERNEL_FLAGS = ("fq_api",)
SINGLE = ("fq_api", "fq_attn_lut", "fq_encode_mfma", "fq_encode_h16", "fq_encode_full", "fq_encode_small", "fq_decode_mfma", "fq_train", "fq_prefill")
ARCH = os.environ.get("FQ_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         # no packed-fp32 instruction forms in any kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(job):
    src, obj, defs = job
    extra = [] if os.path.basename(src)[:-4] in NO_KERNEL_FLAGS else KERNEL_FLAGS
    cmd = [_hipcc(), *FLAGS, *extra, *defs, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    work = []
    for name in PER_K:
        src = os.path.join(CSRC, name + ".hip")
        work.append((src, os.path.join(BUILD, name + ".o"), []))
        for k in KS:
            work.append((src, os.path.join(BUILD, f"{name}_k{k}.o"), [f"-DFQ_ONLY_K={k}"]))
    for name in SINGLE:
        work.append((os.path.join(CSRC, name + ".hip"), os.path.join(BUILD, name + ".o"), []))
    jobs = jobs or min(len(work), max(1, os.cpu_count() or 1))
    # longest first: the k=1 and k=2 encoders dominate
    order = sorted(work, key=lambda w: ("fq_encode_k1" not in w[1], "fq_encode_k2" not in w[1], "encode" not in w[1]))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, order))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", flush=True)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs)
    sys.exit(0)
