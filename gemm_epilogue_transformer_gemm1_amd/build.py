"""Build libcoda.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m gemm_epilogue_transformer_gemm1_amd.build

Every call recompiles all sources (a few seconds each, in parallel) and
writes gemm_epilogue_transformer_gemm1_amd/libcoda.so.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcoda.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["coda_abi.cpp", "gemm_bf16.hip", "gemm_bwd.hip", "gemm_fp8.hip", "gemm_wide.hip",
           "gemm_splitk.hip", "light_kernels.hip", "attention.hip"]
# sources whose kernels run inline-asm MFMAs: their assembly is hazard-checked
MFMA_SOURCES = ["gemm_bf16.hip", "gemm_bwd.hip", "gemm_fp8.hip", "gemm_wide.hip",
                "gemm_splitk.hip", "attention.hip"]

# Packed fp32 VALU forms are kept out of generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcoda)")


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-c",
                                   os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    p = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{errs}")
    return obj, errs


def _check(src):
    from gemm_epilogue_transformer_gemm1_amd import isa_check
    flags = [f for f in HIP_FLAGS if f != "-fPIC"] + ["-I", os.path.join(HERE, "..", "include")]
    return isa_check.check_source(hipcc(), os.path.join(CSRC, src), flags)


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(MFMA_SOURCES))) as ex:
        checks = [ex.submit(_check, s) for s in MFMA_SOURCES]
        results = list(ex.map(_compile, SOURCES))
        for c in checks:
            c.result()  # raises if an accumulator access sits too close to an MFMA
    if verbose:
        for (obj, errs) in results:
            if errs.strip():
                print(errs)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + \
        [o for o, _ in results]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("linking libcoda.so failed:\n" + p.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
