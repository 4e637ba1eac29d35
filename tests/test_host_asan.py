"""The C ABI's argument validation under host AddressSanitizer (CPU only).

capi.hip and qtensor.cpp are rebuilt with their host code instrumented
(-Xarch_host -fsanitize=address: the device code is built as usual and is
never run here), linked with the library's other objects, and driven by
tests/host_asan_driver.c, which makes only calls the library must refuse
before any HIP call and checks each status.  A read or write past any host
buffer the library is handed fails the run.
"""

import os
import shutil
import subprocess

import pytest

from bit_quantized_finetuning_nf4_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(B.BUILD, "asan")
INSTRUMENTED = ["capi.hip", "qtensor.cpp"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _clang():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = os.path.join(rocm, "llvm", "bin", "clang")
    return exe if os.path.exists(exe) else shutil.which("clang")


@pytest.fixture(scope="module")
def driver():
    if _clang() is None:
        pytest.skip("no clang for the host ASan driver")
    others = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s not in INSTRUMENTED]
    if not all(os.path.exists(o) for o in others):
        B.build(verbose=False)
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in INSTRUMENTED:
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run([B.hipcc()] + B.flags() + ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                                        "-Xarch_host", "-fno-omit-frame-pointer",
                                        "-c", os.path.join(B.CSRC, src), "-o", obj])
        objs.append(obj)
    lib = os.path.join(OUT, "libqlora_asan.so")
    _run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib] + objs + others)
    exe = os.path.join(OUT, "host_asan_driver")
    _run([_clang(), "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_asan_driver.c"),
          "-o", exe, "-L", OUT, "-lqlora_asan", f"-Wl,-rpath,{OUT}"])
    return exe


def test_validation_is_clean_under_asan(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host asan driver OK" in r.stdout, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr
