"""Pins of the layer-set group oracle (oracle/group.py) against formulations
other than its own loop over linears:

  * G = 1 is the single linear;
  * the group equals ONE linear on the stacked weight [G N x K] with the
    stacked A [G r x K] and a block-diagonal B [G N x G r] (written out here
    with explicit zero blocks);
  * its gradients are the derivatives of L = <dY, Y>, checked by finite
    differences (exact up to rounding: L is linear in X, and in A or B with
    the other fixed).
"""

import numpy as np
import pytest

import oracle


def _case(G, M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    Wds = [rng.standard_normal((N, K)) * 0.1 for _ in range(G)]
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((G * r, K)) * 0.1
    B = rng.standard_normal((G * N, r)) * 0.1
    dY = rng.standard_normal((M, G * N))
    return Wds, X, A, B, dY


def _block_diag(B, G, N, r):
    Bd = np.zeros((G * N, G * r))
    for g in range(G):
        Bd[g * N:(g + 1) * N, g * r:(g + 1) * r] = B[g * N:(g + 1) * N]
    return Bd


def test_one_linear_is_the_linear_layer():
    Wds, X, A, B, dY = _case(1, 5, 16, 24, 4, 0)
    np.testing.assert_array_equal(oracle.group_fwd(Wds, X, A, B, 8.0), oracle.linear_fwd(Wds[0], X, A, B, 8.0))
    for a, b in zip(oracle.group_bwd(Wds, X, dY, A, B, 8.0), oracle.linear_bwd(Wds[0], X, dY, A, B, 8.0)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("G", [2, 3])
def test_group_is_one_linear_with_a_block_diagonal_adapter(G):
    M, N, K, r, alpha = 7, 16, 24, 4, 8.0
    Wds, X, A, B, dY = _case(G, M, N, K, r, G)
    s = oracle.lora_scale(alpha, r)
    Ws, Bd = np.concatenate(Wds, axis=0), _block_diag(B, G, N, r)
    Y = X @ Ws.T + s * (X @ A.T) @ Bd.T
    np.testing.assert_allclose(oracle.group_fwd(Wds, X, A, B, alpha), Y, rtol=1e-12, atol=1e-12)
    dX, dA, dB = oracle.group_bwd(Wds, X, dY, A, B, alpha)
    np.testing.assert_allclose(dX, dY @ Ws + s * (dY @ Bd) @ A, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, s * (dY @ Bd).T @ X, rtol=1e-12, atol=1e-12)
    dBd = s * dY.T @ (X @ A.T)          # gradient of every entry of the block-diagonal B
    for g in range(G):                  # only the diagonal blocks are parameters
        np.testing.assert_allclose(dB[g * N:(g + 1) * N], dBd[g * N:(g + 1) * N, g * r:(g + 1) * r],
                                   rtol=1e-12, atol=1e-12)


def test_gradients_are_finite_differences_of_the_loss():
    G, M, N, K, r, alpha = 3, 4, 8, 16, 2, 4.0
    Wds, X, A, B, dY = _case(G, M, N, K, r, 7)
    loss = lambda X_, A_, B_: float(np.sum(dY * oracle.group_fwd(Wds, X_, A_, B_, alpha)))
    dX, dA, dB = oracle.group_bwd(Wds, X, dY, A, B, alpha)
    L0, eps = loss(X, A, B), 1e-3
    for (i, j) in [(0, 0), (3, 15), (2, 7)]:
        E = np.zeros_like(X)
        E[i, j] = eps
        assert abs((loss(X + E, A, B) - L0) / eps - dX[i, j]) < 1e-8
    for (i, j) in [(0, 0), (5, 3), (2, 11)]:   # rows of different adapters
        E = np.zeros_like(A)
        E[i, j] = eps
        assert abs((loss(X, A + E, B) - L0) / eps - dA[i, j]) < 1e-8
    for (i, j) in [(0, 1), (9, 0), (23, 1)]:
        E = np.zeros_like(B)
        E[i, j] = eps
        assert abs((loss(X, A, B + E) - L0) / eps - dB[i, j]) < 1e-8


def test_without_adapters():
    Wds, X, _, _, dY = _case(2, 3, 8, 16, 2, 3)
    np.testing.assert_allclose(oracle.group_fwd(Wds, X), X @ np.concatenate(Wds).T, rtol=1e-13)
    dX, dA, dB = oracle.group_bwd(Wds, X, dY)
    np.testing.assert_allclose(dX, dY @ np.concatenate(Wds), rtol=1e-13)
    assert dA is None and dB is None
