"""GPU parity of qlora_linear_fwd_noalloc (the forward without a workspace
argument, for callers that cannot allocate) against qlora_linear_fwd.

The no-allocation call always takes the fused path (its 32 MiB array cannot
hold a bf16 weight), so the reference is qlora_linear_fwd with a workspace
sized for the fused path: the same kernels, compared bit for bit, and both
within the forward tolerances of the fp64 oracle.  Two calls in a row, the
second on a smaller input; U comes back as well.  Then a rank-0 call (no
scratch needed) and a call that keeps U in the array only.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _case(N, K, M, r, seed):
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    return dict(W=g((N, K), 0.02), X=g((M, K), 1.0), A=g((r, K), 0.2) if r else None,
                B=g((N, r), 0.2) if r else None, alpha=16.0)


def _oracle_y(d):
    c, a, s = oracle.quantize(d["W"])
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size)).reshape(d["W"].shape)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    return oracle.linear_fwd(Wd, f("X"), f("A"), f("B"), d["alpha"])


def _check(d, label):
    print(f"[noalloc] {label}", flush=True)
    q = ops.quantize(bits_to_torch(d["W"]))
    X = bits_to_torch(d["X"])
    A = None if d["A"] is None else bits_to_torch(d["A"])
    B = None if d["B"] is None else bits_to_torch(d["B"])
    r = 0 if A is None else A.shape[0]
    Yn, Un = ops.linear_fwd_noalloc(q, X, A, B, d["alpha"], save_u=True)
    Yw, Uw = ops.linear_fwd(q, X, A, B, d["alpha"], save_u=True, path="fused")
    torch.cuda.synchronize()
    assert torch.equal(Yn.view(torch.int16), Yw.view(torch.int16)), f"{label}: Y differs from qlora_linear_fwd"
    if r:
        assert torch.equal(Un.view(torch.int16), Uw.view(torch.int16)), f"{label}: U differs"
    assert_close(torch_to_f64(Yn), _oracle_y(d), f"{label} Y")
    return q, X, A, B


def test_two_calls_in_a_row_second_smaller():
    _check(_case(1024, 1024, 256, 8, seed=900), "call 1: N1024 K1024 M256 r8")
    _check(_case(264, 320, 100, 16, seed=901), "call 2: N264 K320 M100 r16")


def test_largest_rank_and_no_adapter():
    # r = 128 at M = 4096 uses about 17 MiB of the array; r = 0 uses none
    _check(_case(512, 8192, 4096, 128, seed=902), "N512 K8192 M4096 r128")
    _check(_case(256, 512, 300, 0, seed=903), "N256 K512 M300 r0")


def test_u_is_recomputed_into_scratch_when_not_saved():
    # without U_save, U lives in the array; the result must not depend on it
    d = _case(768, 2048, 512, 64, seed=904)
    q, X, A, B = _check(d, "N768 K2048 M512 r64 (saved U)")
    Y1 = ops.linear_fwd_noalloc(q, X, A, B, d["alpha"])
    Y2 = ops.linear_fwd(q, X, A, B, d["alpha"], path="fused")
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


def test_oversize_call_is_rejected():
    d = _case(64, 8192, 8, 8, seed=905)
    q = ops.quantize(bits_to_torch(d["W"]))
    # M = 65536 at r = 128 needs more than the array: rejected before launch
    # (the tensors are never touched, so small ones stand in)
    X = torch.empty(8, 8192, dtype=torch.bfloat16, device="cuda")
    A = torch.empty(128, 8192, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(64, 128, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(8, 64, dtype=torch.bfloat16, device="cuda")
    from bit_quantized_finetuning_nf4_amd._lib import lib
    import ctypes
    desc = q.desc()
    st = lib().qlora_linear_fwd_noalloc(ctypes.byref(desc), ctypes.c_void_p(X.data_ptr()), 65536,
                                        ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()), 128, 16.0,
                                        ctypes.c_void_p(Y.data_ptr()), None, None)
    assert st == 5   # QLORA_E_WORKSPACE
