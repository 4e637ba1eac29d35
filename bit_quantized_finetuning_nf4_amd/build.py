"""Build libqlora.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m bit_quantized_finetuning_nf4_amd.build

Objects go to ``_build/`` next to this file; the shared library is written
to ``libqlora.so`` in the package directory, where the binding loads it.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlora.so")
SOURCES = ["quantize.hip", "gemm.hip", "gemm_nf4.hip", "gemm_bf16.hip", "gemv.hip", "optim.hip", "paged.hip", "capi.hip", "qtensor.cpp"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "bin", "hipcc")
    return exe if os.path.exists(exe) else (shutil.which("hipcc") or "hipcc")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-Wall", "-Wno-unused-command-line-argument",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj, errs


def build(verbose=True):
    """Compile every HIP source for gfx950 and link libqlora.so; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, errs) in results:
        if errs and verbose:
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
