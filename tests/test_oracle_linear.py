"""Pins for the oracle's fp64 forward / backward / GEMV (CPU only).

Pinned against: element-by-element pure-Python sums on tiny shapes, central
finite differences of the scalar <dY, Y> (which checks every gradient
against the forward, including the scale s and the operand orientation),
the merged-weight identity of LoRA (W + s B A, deepfa.ir "LoRA:
Prerequisite"), the special cases W = 0 and A = 0, and GEMV = forward at
one token.
"""

import itertools

import numpy as np
import pytest

import oracle


def _tiny(seed, M=3, N=5, K=4, r=2):
    rng = np.random.default_rng(seed)
    return dict(W=rng.standard_normal((N, K)), X=rng.standard_normal((M, K)),
                A=rng.standard_normal((r, K)), B=rng.standard_normal((N, r)),
                dY=rng.standard_normal((M, N)), alpha=3.0)


def test_lora_scale():
    assert oracle.lora_scale(16, 8) == 2.0
    assert oracle.lora_scale(16, 64) == 0.25
    assert oracle.lora_scale(1.0, 3) == float(np.float32(1.0 / 3.0))
    assert oracle.lora_scale(16, 0) == 0.0


def test_forward_elementwise_sums():
    t = _tiny(0)
    W, X, A, B = t["W"], t["X"], t["A"], t["B"]
    s = oracle.lora_scale(t["alpha"], 2)
    Y = oracle.linear_fwd(W, X, A, B, t["alpha"])
    M, K = X.shape
    N, r = B.shape
    for m, n in itertools.product(range(M), range(N)):
        base = sum(X[m][k] * W[n][k] for k in range(K))
        lora = sum(B[n][j] * sum(X[m][k] * A[j][k] for k in range(K)) for j in range(r))
        assert abs(Y[m, n] - (base + s * lora)) < 1e-12


def test_gemv_elementwise_and_equals_forward_at_one_token():
    t = _tiny(1, M=1)
    W, x, A, B = t["W"], t["X"][0], t["A"], t["B"]
    s = oracle.lora_scale(t["alpha"], 2)
    y = oracle.gemv(W, x, A, B, t["alpha"])
    for n in range(W.shape[0]):
        u = [sum(A[j][k] * x[k] for k in range(len(x))) for j in range(A.shape[0])]
        ref = sum(W[n][k] * x[k] for k in range(len(x))) + s * sum(B[n][j] * u[j] for j in range(len(u)))
        assert abs(y[n] - ref) < 1e-12
    assert np.allclose(y, oracle.linear_fwd(W, x[None, :], A, B, t["alpha"])[0], rtol=0, atol=1e-13)


def _objective(W, X, A, B, dY, alpha):
    return float(np.sum(dY * oracle.linear_fwd(W, X, A, B, alpha)))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_central_finite_differences(seed):
    t = _tiny(seed, M=4, N=6, K=5, r=3)
    W, X, A, B, dY, al = t["W"], t["X"], t["A"], t["B"], t["dY"], t["alpha"]
    dX, dA, dB = oracle.linear_bwd(W, X, dY, A, B, al)
    h = 1e-6
    for name, P, G in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        num = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + h
            fp = _objective(W, X, A, B, dY, al)
            P[idx] = old - h
            fm = _objective(W, X, A, B, dY, al)
            P[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(G, num, rtol=1e-6, atol=1e-7), name


def test_lora_equals_merged_weight():
    t = _tiny(2)
    s = oracle.lora_scale(t["alpha"], 2)
    merged = t["W"] + s * t["B"] @ t["A"]
    Y = oracle.linear_fwd(t["W"], t["X"], t["A"], t["B"], t["alpha"])
    assert np.allclose(Y, oracle.linear_fwd(merged, t["X"]), rtol=0, atol=1e-12)
    dX, _, _ = oracle.linear_bwd(t["W"], t["X"], t["dY"], t["A"], t["B"], t["alpha"])
    dXm, _, _ = oracle.linear_bwd(merged, t["X"], t["dY"])
    assert np.allclose(dX, dXm, rtol=0, atol=1e-12)


def test_special_cases_reduce_to_plain_products():
    t = _tiny(3)
    s = oracle.lora_scale(t["alpha"], 2)
    Z = np.zeros_like(t["W"])
    # W = 0: pure LoRA
    Y = oracle.linear_fwd(Z, t["X"], t["A"], t["B"], t["alpha"])
    assert np.allclose(Y, s * t["X"] @ t["A"].T @ t["B"].T, rtol=0, atol=1e-12)
    # A = 0: plain product, and dB = 0 while dA still flows through B
    A0 = np.zeros_like(t["A"])
    Y = oracle.linear_fwd(t["W"], t["X"], A0, t["B"], t["alpha"])
    assert np.allclose(Y, t["X"] @ t["W"].T, rtol=0, atol=1e-12)
    dX, dA, dB = oracle.linear_bwd(t["W"], t["X"], t["dY"], A0, t["B"], t["alpha"])
    assert np.allclose(dX, t["dY"] @ t["W"], rtol=0, atol=1e-12)
    assert np.all(dB == 0) and np.any(dA != 0)
    # r = 0: base layer only
    dX, dA, dB = oracle.linear_bwd(t["W"], t["X"], t["dY"])
    assert dA is None and dB is None


def test_adjoint_identity_in_x():
    t = _tiny(4, M=7, N=9, K=6, r=3)
    Y = oracle.linear_fwd(t["W"], t["X"], t["A"], t["B"], t["alpha"])
    dX, _, _ = oracle.linear_bwd(t["W"], t["X"], t["dY"], t["A"], t["B"], t["alpha"])
    # Y is linear in X, so <dY, Y(X)> = <dX, X>
    assert abs(np.sum(t["dY"] * Y) - np.sum(dX * t["X"])) < 1e-10
