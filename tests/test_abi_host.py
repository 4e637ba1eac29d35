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


def test_dense_split_workspace(L):
    """The dense dX product splits its contraction only for shapes with at
    most 128 output tiles of 256 x 256 and a contraction of 16384 columns or
    more; the workspace holds the two fp32 partials."""
    op = _lib.QLORA_OP_BF16_DX
    # the 7B gate/up group: dX [2048 x 4096] over 2 x 11008 columns
    assert L.qlora_workspace_bytes(op, 2048, 11008, 4096, 64, 2) == 2 * 2048 * 4096 * 4
    # each linear alone (11008 columns), q/k/v (12288), 65B shapes (512 tiles): no split
    assert L.qlora_workspace_bytes(op, 2048, 11008, 4096, 64, 1) == 0
    assert L.qlora_workspace_bytes(op, 2048, 4096, 4096, 64, 3) == 0
    assert L.qlora_workspace_bytes(op, 4096, 22016, 8192, 64, 2) == 0
    # the group backward's workspace has the partials beside deq(W)^T
    with_split = L.qlora_workspace_bytes(_lib.QLORA_OP_GROUP_BWD, 2048, 11008, 4096, 64, 2)
    dq = 2 * 11008 * 4096 * 2
    assert with_split >= dq + 2 * 2048 * 4096 * 4


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


def test_lora_side_products_reject_32_bit_overflow(L):
    """The LoRA products address a 128-row tile of X or dY and the rank-side
    operand with 32-bit byte ranges: a K or N of 2^24 or more is refused
    before any launch (one token, so the token-matrix limits pass)."""
    fake = ctypes.c_void_p(4096)
    big = 1 << 24
    assert L.qlora_lora_down(fake, fake, 1, big, 64, fake, fake, 1 << 30, None) == 4
    assert L.qlora_lora_down(fake, fake, 1, big - 8, 64, fake, None, 0, None) != 4
    assert L.qlora_lora_dy_b(fake, fake, 1, big, 64, fake, fake, 1 << 30, None) == 4
    wide = _desc(rows=8, cols=big, codes=4096, aq=8192, s2=12288)
    assert L.qlora_linear_fwd(ctypes.byref(wide), fake, 1, fake, fake, 64, 16.0, fake, None, fake, 1 << 40,
                              None) == 4
    assert L.qlora_linear_bwd(ctypes.byref(wide), fake, fake, 1, fake, fake, 64, 16.0, None, fake, fake, fake,
                              fake, 1 << 40, None) == 4
    tall = _desc(rows=big, cols=64, codes=4096, aq=8192, s2=12288)
    assert L.qlora_linear_bwd(ctypes.byref(tall), fake, fake, 1, fake, fake, 64, 16.0, None, fake, fake, fake,
                              fake, 1 << 40, None) == 4


def test_noalloc_forward_rejects_oversize_and_bad_arguments_on_the_host(L):
    """qlora_linear_fwd_noalloc: the same checks as qlora_linear_fwd, and a
    call whose scratch exceeds the static array is refused before anything
    touches the GPU."""
    fake = ctypes.c_void_p(4096)
    d = _desc(rows=1024, cols=8192, codes=4096, aq=8192, s2=12288)
    need = L.qlora_workspace_bytes(0, 65536, 1024, 8192, 128, 0)
    assert need > _lib.STATIC_SCRATCH_BYTES
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, 65536, fake, fake, 128, 16.0, fake, None, None) == 5
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), None, 4, None, None, 0, 0.0, fake, None, None) == 1
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, 4, fake, fake, 12, 1.0, fake, None, None) == 4
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), ctypes.c_void_p(4098), 4, None, None, 0, 0.0, fake, None,
                                      None) == 2
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(d), fake, 0, None, None, 0, 0.0, fake, None, None) == 3


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


def _paged(L, sizes, budget):
    from bit_quantized_finetuning_nf4_amd._lib import PagedLayoutDesc, PagedTensorDesc
    descs = (PagedTensorDesc * len(sizes))()
    for i, n in enumerate(sizes):
        descs[i] = PagedTensorDesc(4096, None, 4096, 4096, 4096, n)   # never dereferenced
    lay = PagedLayoutDesc()
    st = L.qlora_paged_layout_of(descs, len(sizes), budget, ctypes.byref(lay))
    return st, lay


def test_paged_optimizer_layout_policy(L):
    """The paging policy is host arithmetic: everything resident when the
    moments fit; otherwise two staging slots and the longest prefix of
    tensors whose moments fit the rest, never more than the budget."""
    sizes = [4096, 5, 64, 700, 300000, 1000003]
    state = lambda n: 2 * (-(-4 * n // 256) * 256)            # m and v, 256-byte aligned each
    total = sum(state(n) for n in sizes)
    st, lay = _paged(L, sizes, total)
    assert st == 0 and lay.resident == len(sizes) and lay.chunk == 0 and lay.staging_bytes == 0
    for budget in (total - 1, total // 2, 1 << 20, 65536, 2048):
        st, lay = _paged(L, sizes, budget)
        assert st == 0, budget
        assert 64 <= lay.chunk <= (4 << 20) and lay.chunk % 64 == 0
        assert lay.staging_bytes == 2 * state(lay.chunk)
        assert lay.staging_bytes + lay.resident_bytes <= budget
        assert lay.resident_bytes == sum(state(n) for n in sizes[:lay.resident])
        if lay.resident < len(sizes):   # the prefix is as long as the budget allows
            assert lay.staging_bytes + lay.resident_bytes + state(sizes[lay.resident]) > budget
    assert _paged(L, sizes, 2047)[0] == 5                      # not even two minimal slots
    assert _paged(L, [0], 1 << 20)[0] == 3
    fake = ctypes.c_void_p(4096)
    from bit_quantized_finetuning_nf4_amd._lib import PagedTensorDesc
    d = (PagedTensorDesc * 1)(PagedTensorDesc(4096, None, 4096, 4096, 4096, 1000))
    assert L.qlora_paged_adamw(d, 1, fake, 1 << 20, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, 0, None, None) == 3   # step 0
    assert L.qlora_paged_adamw(d, 1, fake, 1 << 20, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, 0, None, None) == 3   # beta1 1
    assert L.qlora_paged_adamw(d, 1, ctypes.c_void_p(4096 + 16), 1 << 20, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0, None,
                               None) == 2                                                            # ws alignment
    assert L.qlora_paged_adamw(d, 1, fake, 512, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0, None, None) in (0, 5)


def test_group_calls_validate_on_the_host(L):
    """Layer-set groups: workspace sizes and every rejection happen on the
    host, before anything is enqueued (fake, never-dereferenced addresses)."""
    fwd1 = L.qlora_workspace_bytes(0, 4096, 8192, 8192, 64, 0)   # one linear, staged
    gf = L.qlora_workspace_bytes(6, 4096, 8192, 8192, 64, 3)
    gb = L.qlora_workspace_bytes(7, 4096, 8192, 8192, 64, 3)
    assert gf >= 3 * 8192 * 8192 * 2 + 4096 * 192 * 2 and gf > fwd1
    assert gb >= 3 * 8192 * 8192 * 2 + 2 * 4096 * 192 * 2
    assert L.qlora_workspace_bytes(6, 4096, 8192, 8192, 0, 2) == 2 * 8192 * 8192 * 2   # no adapter: the stack only
    assert L.qlora_workspace_bytes(6, 4096, 8192, 8192, 64, 0) == 0      # G >= 1
    assert L.qlora_workspace_bytes(6, 4096, 8192, 8192, 64, 5) == 0      # G r > 256
    assert L.qlora_workspace_bytes(7, 4096, 1 << 16, 1 << 16, 8, 1) == 0  # G N K >= 2^31

    fake = ctypes.c_void_p(4096)
    big = 1 << 40
    W = lambda *ds: (Nf4WeightDesc * len(ds))(*ds)
    three = W(_desc(128, 64), _desc(128, 64), _desc(128, 64))
    gf = lambda w, g, x, m, a, b, r, y, ws=fake, n=big: L.qlora_group_fwd(w, g, x, m, a, b, r, 16.0, y, None, ws, n,
                                                                          None)
    assert gf(None, 3, fake, 4, fake, fake, 16, fake) == 1
    assert gf(three, 0, fake, 4, fake, fake, 16, fake) == 3                          # G >= 1
    assert gf(W(_desc(128, 64), _desc(192, 64)), 2, fake, 4, fake, fake, 16, fake) == 3   # shapes differ
    assert gf(W(_desc(72, 64), _desc(72, 64)), 2, fake, 4, fake, fake, 16, fake) == 4     # N % 64
    assert gf(three, 3, fake, 4, fake, fake, 96, fake) == 4                          # G r = 288 > 256
    assert gf(three, 3, fake, 4, fake, fake, 12, fake) == 4                          # r % 8
    assert gf(three, 3, fake, 4, None, fake, 16, fake) == 1                          # A missing
    assert gf(three, 3, None, 4, fake, fake, 16, fake) == 1
    assert gf(three, 3, fake, 0, fake, fake, 16, fake) == 3                          # M >= 1
    assert gf(three, 3, ctypes.c_void_p(4098), 4, fake, fake, 16, fake) == 2         # X alignment
    assert gf(three, 3, fake, 4, fake, fake, 16, fake, n=16) == 5                    # workspace too small
    assert gf(three, 3, fake, 4, fake, fake, 16, fake, ws=None) == 1                 # workspace missing
    gb = lambda w, g, m, r, dx, da, db, n=big: L.qlora_group_bwd(w, g, fake, fake, m, fake if r else None,
                                                                 fake if r else None, r, 16.0, None, dx, da, db,
                                                                 fake, n, None)
    assert gb(three, 3, 4, 16, fake, None, fake) == 1                                # dA missing
    assert gb(three, 3, 4, 0, fake, fake, None) == 3                                 # no adapter, no dA
    assert gb(three, 3, 4, 16, fake, fake, fake, n=16) == 5
    assert gb(W(_desc(128, 64), _desc(128, 128)), 2, 4, 16, fake, fake, fake) == 3


def test_group_building_blocks_validate_on_the_host(L):
    fake, big = ctypes.c_void_p(4096), 1 << 40
    W = lambda *ds: (Nf4WeightDesc * len(ds))(*ds)
    two = W(_desc(128, 64), _desc(128, 64))
    assert L.qlora_group_dequant(None, 2, fake, None) == 1
    assert L.qlora_group_dequant(two, 0, fake, None) == 3
    assert L.qlora_group_dequant(two, 2, None, None) == 1
    assert L.qlora_group_dequant_t(two, 2, ctypes.c_void_p(4100), None) == 2
    assert L.qlora_group_dequant_t(W(_desc(128, 64), _desc(64, 64)), 2, fake, None) == 3
    # dense products: G N K, N % 64, ranks
    assert L.qlora_bf16_group_fwd(fake, 0, 128, 64, fake, 4, None, None, 0, 0.0, fake, None) == 3
    assert L.qlora_bf16_group_fwd(fake, 2, 72, 64, fake, 4, None, None, 0, 0.0, fake, None) == 4
    assert L.qlora_bf16_group_fwd(fake, 3, 128, 64, fake, 4, fake, fake, 96, 16.0, fake, None) == 4
    assert L.qlora_bf16_group_fwd(fake, 2, 128, 64, fake, 4, None, fake, 16, 16.0, fake, None) == 1
    assert L.qlora_bf16_group_fwd(fake, 2, 1 << 16, 1 << 15, fake, 4, None, None, 0, 0.0, fake, None) == 4
    assert L.qlora_bf16_group_dx(fake, 2, 128, 64, fake, 4, fake, None, 16, 16.0, fake, None, 0, None) == 1
    assert L.qlora_bf16_group_dx(None, 2, 128, 64, fake, 4, None, None, 0, 0.0, fake, None, 0, None) == 1
    # a workspace must be 16-byte aligned
    assert L.qlora_bf16_group_dx(fake, 2, 128, 64, fake, 4, None, None, 0, 0.0, fake, ctypes.c_void_p(4100), 64,
                                 None) == 2
    # side products
    assert L.qlora_group_lora_dy_b(fake, fake, 4, 128, 16, 2, fake, fake, 16, None) == 5
    assert L.qlora_group_lora_dy_b(fake, fake, 4, 128, 136, 2, fake, fake, big, None) == 4     # r > 128
    assert L.qlora_group_lora_dy_b(fake, fake, 4, 128, 128, 3, fake, fake, big, None) == 4     # G r > 256
    assert L.qlora_group_lora_dy_b(fake, fake, 4, 128, 16, 0, fake, fake, big, None) == 3
    assert L.qlora_group_lora_grads(fake, fake, fake, fake, 4, 128, 64, 16, 2, 16.0, fake, fake, fake, 16,
                                    None) == 5
    assert L.qlora_group_lora_grads(fake, fake, None, fake, 4, 128, 64, 16, 2, 16.0, fake, fake, fake, big,
                                    None) == 1
    assert L.qlora_group_lora_grads(fake, fake, fake, fake, 1 << 20, 1 << 12, 64, 16, 2, 16.0, fake, fake, fake,
                                    big, None) == 4                                            # M G N >= 2^31
    # lora_down takes a group's stacked adapters (rank up to 256)
    assert L.qlora_workspace_bytes(3, 4096, 64, 8192, 192, 0) > 0
    assert L.qlora_workspace_bytes(3, 4096, 64, 8192, 264, 0) == 0
    assert L.qlora_lora_down(fake, fake, 4, 64, 264, fake, fake, big, None) == 4
    assert L.qlora_lora_down(fake, fake, 4, 64, 192, fake, fake, 16, None) == 5
    assert L.qlora_workspace_bytes(8, 4096, 8192, 8192, 64, 3) >= L.qlora_workspace_bytes(3, 4096, 64, 8192, 192, 0)
