"""Host-side tests of the C ABI (CPU only: no kernel is launched).

The library must load, export every function include/qlora.h declares,
return its own NF4 table bit-identical to the oracle's, size buffers by the
storage formula, and reject bad arguments before touching the GPU.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_nf4_amd import _lib
from bit_quantized_finetuning_nf4_amd._lib import Nf4WeightDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libqlora.so is not built (run python -m bit_quantized_finetuning_nf4_amd.build)")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_operations():
    fns = declared_functions()
    for f in ("qlora_quantize", "qlora_dequant", "qlora_linear_fwd", "qlora_linear_bwd", "qlora_gemv"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    fns = declared_functions()
    assert sorted(_lib.EXPORTS) == fns
    for f in fns:
        assert hasattr(L, f), f


def test_nf4_table_bitwise_equals_oracle(L):
    buf = (ctypes.c_float * 16)()
    L.qlora_nf4_levels(buf)
    got = np.array(list(buf), dtype=np.float32).view(np.uint32)
    assert np.array_equal(got, oracle.nf4_levels().view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(1, 1), (1024, 1024), (22016, 8192), (3, 1000), (7, 9)])
def test_sizes_match_storage_formula(L, rows, cols):
    c, a, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qlora_sizes(rows, cols, 64, 256, ctypes.byref(c), ctypes.byref(a), ctypes.byref(s)) == 0
    assert (c.value, a.value, s.value) == oracle.storage_sizes(rows * cols)


def test_sizes_rejects_bad_arguments(L):
    assert L.qlora_sizes(0, 5, 64, 256, None, None, None) == 3
    assert L.qlora_sizes(5, -1, 64, 256, None, None, None) == 3
    assert L.qlora_sizes(5, 5, 32, 256, None, None, None) == 4
    assert L.qlora_sizes(5, 5, 64, 128, None, None, None) == 4


def test_status_strings_and_version(L):
    for code in range(7):
        assert L.qlora_status_str(code).decode().startswith(_lib.STATUS_NAMES[code])
    assert L.qlora_version().decode().count(".") == 2


def test_workspace_query(L):
    assert L.qlora_workspace_bytes(0, 256, 1024, 1024, 0, 0) == 0
    assert L.qlora_workspace_bytes(1, 256, 1024, 1024, 0, 0) == 0
    fwd = L.qlora_workspace_bytes(0, 4096, 8192, 8192, 64, 0)
    bwd = L.qlora_workspace_bytes(1, 4096, 8192, 8192, 64, 0)
    assert fwd >= 4096 * 64 * 2 and bwd >= 2 * 4096 * 64 * 2
    # GEMV: u = A x per job plus the device job table; N is the largest row count
    gv = L.qlora_workspace_bytes(2, 0, 22016, 8192, 64, 560)
    assert gv >= 560 * 128 * 4 + 560 * 72
    assert L.qlora_workspace_bytes(2, 0, 0, 0, 0, 560) == 0       # N required
    assert L.qlora_workspace_bytes(0, 0, 8, 8, 16, 0) == 0       # invalid -> 0


def _desc(rows=64, cols=64, bs=64, g=256, codes=16, aq=16, s2=16):
    return Nf4WeightDesc(rows, cols, bs, g, codes, aq, s2)


def test_validation_happens_before_any_launch(L):
    # fake, never-dereferenced addresses: every call must fail validation
    # on the host and return without touching the GPU
    fake = ctypes.c_void_p(4096)
    d = _desc(codes=4096, aq=8192, s2=12288)
    assert L.qlora_quantize(None, ctypes.byref(d), None) == 1
    assert L.qlora_quantize(ctypes.c_void_p(4098), ctypes.byref(d), None) == 2
    assert L.qlora_quantize(fake, None, None) == 1
    bad = _desc(bs=32, codes=4096, aq=8192, s2=12288)
    assert L.qlora_quantize(fake, ctypes.byref(bad), None) == 4
    neg = _desc(rows=0, codes=4096, aq=8192, s2=12288)
    assert L.qlora_dequant(ctypes.byref(neg), fake, None) == 3
    nul = _desc(codes=0, aq=8192, s2=12288)
    assert L.qlora_dequant(ctypes.byref(nul), fake, None) == 1
    # GEMM paths need cols % 64 == 0 and rows % 8 == 0
    odd = _desc(rows=64, cols=96, codes=4096, aq=8192, s2=12288)
    assert L.qlora_linear_fwd(ctypes.byref(odd), fake, 4, None, None, 0, 0.0, fake, None, None, 0, None) == 4
    odd = _desc(rows=60, cols=64, codes=4096, aq=8192, s2=12288)
    assert L.qlora_linear_fwd(ctypes.byref(odd), fake, 4, None, None, 0, 0.0, fake, None, None, 0, None) == 4
    # rank must be a multiple of 8 in [0, 128]; A and B required when r > 0
    assert L.qlora_linear_fwd(ctypes.byref(d), fake, 4, fake, fake, 12, 1.0, fake, None, None, 0, None) == 4
    assert L.qlora_linear_fwd(ctypes.byref(d), fake, 4, fake, fake, 144, 1.0, fake, None, None, 0, None) == 4
    assert L.qlora_linear_fwd(ctypes.byref(d), fake, 4, None, fake, 16, 1.0, fake, None, None, 0, None) == 1
    # workspace too small
    assert L.qlora_linear_fwd(ctypes.byref(d), fake, 4, fake, fake, 16, 1.0, fake, None, fake, 16, None) == 5
    assert L.qlora_linear_fwd(ctypes.byref(d), fake, 0, None, None, 0, 0.0, fake, None, None, 0, None) == 3
    # backward: adapter gradients without an adapter, missing outputs
    assert L.qlora_linear_bwd(ctypes.byref(d), fake, fake, 4, None, None, 0, 0.0, None, fake, fake, None,
                              None, 0, None) == 3
    assert L.qlora_linear_bwd(ctypes.byref(d), fake, fake, 4, fake, fake, 16, 1.0, None, fake, None, fake,
                              fake, 1 << 30, None) == 1
    # gemv: empty / oversized job lists, bad rank
    assert L.qlora_gemv(None, 1, None, 0, None) == 1
    job = _lib.GemvJobDesc(ctypes.pointer(d), 4096, None, None, 0, 0.0, 4096)
    jobs = (_lib.GemvJobDesc * 1)(job)
    assert L.qlora_gemv(jobs, 0, None, 0, None) == 3
    assert L.qlora_gemv(jobs, 5000, None, 0, None) == 4
    assert L.qlora_gemv(jobs, 1, None, 0, None) == 1             # the job table needs a workspace
    assert L.qlora_gemv(jobs, 1, fake, 16, None) == 5             # too small for it
    wide = _desc(rows=64, cols=32768 + 64, codes=4096, aq=8192, s2=12288)
    jobs[0].W = ctypes.pointer(wide)
    assert L.qlora_gemv(jobs, 1, fake, 1 << 20, None) == 4        # x is staged whole in LDS
    jobs[0].W = ctypes.pointer(d)
    # prepared calls: a plan is required, and an unfilled plan is refused
    plan = _lib.GemvPlanDesc()
    assert L.qlora_gemv_prepare(jobs, 1, fake, 1 << 20, None, None) == 1
    assert L.qlora_gemv_prepare(jobs, 1, fake, 16, ctypes.byref(plan), None) == 5
    assert L.qlora_gemv_run(None, None) == 1
    assert L.qlora_gemv_run(ctypes.byref(plan), None) == 3
    jobs[0].r = 16
    assert L.qlora_gemv(jobs, 1, None, 0, None) == 1


@pytest.mark.parametrize("name,cb", [("nf4", 0), ("fp4", 1), ("int4", 2)])
def test_codebook_tables_bitwise_equal_oracle(L, name, cb):
    buf = (ctypes.c_float * 16)()
    assert L.qlora_codebook_levels(cb, buf) == 0
    got = np.array(list(buf), dtype=np.float32).view(np.uint32)
    assert np.array_equal(got, oracle.codebook_levels(name).view(np.uint32))


def test_codebook_calls_reject_bad_arguments_on_the_host(L):
    buf = (ctypes.c_float * 16)()
    assert L.qlora_codebook_levels(3, buf) == 4
    assert L.qlora_codebook_levels(-1, buf) == 4
    assert L.qlora_codebook_levels(0, None) == 1
    fake = ctypes.c_void_p(4096)
    d = _desc(codes=4096, aq=8192, s2=12288)
    for cb in (3, -1, 100):
        d.codebook = cb
        assert L.qlora_quantize(fake, ctypes.byref(d), None) == 4
        assert L.qlora_dequant(ctypes.byref(d), fake, None) == 4
        assert L.qlora_linear_fwd(ctypes.byref(d), fake, 4, None, None, 0, 0.0, fake, None, None, 0, None) == 4


def test_gemv_rejects_mixed_codebooks_on_the_host(L):
    d0 = _desc(codes=4096, aq=8192, s2=12288)
    d1 = _desc(codes=4096, aq=8192, s2=12288)
    d1.codebook = 2
    jobs = (_lib.GemvJobDesc * 2)(_lib.GemvJobDesc(ctypes.pointer(d0), 4096, None, None, 0, 0.0, 4096),
                                   _lib.GemvJobDesc(ctypes.pointer(d1), 4096, None, None, 0, 0.0, 4096))
    assert L.qlora_gemv(jobs, 2, ctypes.c_void_p(4096), 1 << 20, None) == 4



def test_gemv_token_counts_on_the_host(L):
    # m < 0 is a shape error, m > 16 unsupported; the workspace grows with the
    # largest m, and a workspace sized for one token is too small for sixteen
    d = _desc(codes=4096, aq=8192, s2=12288)
    fake = ctypes.c_void_p(4096)
    job = _lib.GemvJobDesc(ctypes.pointer(d), 4096, None, None, 0, 0.0, 4096, 1)
    jobs = (_lib.GemvJobDesc * 1)(job)
    op = _lib.QLORA_OP_GEMV
    one = L.qlora_workspace_bytes(op, 1, 64, 64, 0, 1)
    assert L.qlora_workspace_bytes(op, 0, 64, 64, 0, 1) == one
    assert L.qlora_workspace_bytes(op, 16, 64, 64, 0, 1) > one
    assert L.qlora_workspace_bytes(op, 17, 64, 64, 0, 1) == 0
    assert L.qlora_workspace_bytes(op, -1, 64, 64, 0, 1) == 0
    jobs[0].m = -1
    assert L.qlora_gemv(jobs, 1, fake, 1 << 20, None) == 3
    jobs[0].m = 17
    assert L.qlora_gemv(jobs, 1, fake, 1 << 20, None) == 4
    jobs[0].m = 16
    assert L.qlora_gemv(jobs, 1, fake, one, None) == 5
    plan = _lib.GemvPlanDesc()
    assert L.qlora_gemv_prepare(jobs, 1, fake, one, ctypes.byref(plan), None) == 5

def test_adamw_rejects_bad_arguments_on_the_host(L):
    f = ctypes.c_void_p(4096)
    a = lambda **k: L.qlora_adamw(k.get("p", f), k.get("pb", None), k.get("g", f), k.get("m", f), k.get("v", f),
                                  k.get("n", 8), k.get("lr", 1e-3), k.get("b1", 0.9), k.get("b2", 0.999),
                                  k.get("eps", 1e-8), k.get("wd", 0.0), k.get("t", 1), None)
    assert a(p=None) == 1 and a(g=None) == 1 and a(m=None) == 1 and a(v=None) == 1
    assert a(p=ctypes.c_void_p(4100)) == 2 and a(pb=ctypes.c_void_p(4098)) == 2
    assert a(n=0) == 3 and a(t=0) == 3 and a(b1=1.0) == 3 and a(b2=-0.1) == 3 and a(eps=0.0) == 3
    assert a(lr=float("nan")) == 3 and a(wd=float("inf")) == 3
