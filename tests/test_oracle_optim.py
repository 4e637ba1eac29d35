"""Pins for the oracle's AdamW step (CPU only), by closed forms of special
cases: the first step from zero moments, a constant gradient over many
steps, pure weight decay, and momentum-free (beta = 0) steps."""

import numpy as np

import oracle


def test_first_step_from_zero_moments():
    # m = (1-b1) g and v = (1-b2) g^2, so the corrected moments are g and g^2
    # and the step is lr (g / (|g| + eps) + wd p)
    rng = np.random.default_rng(0)
    p, g = rng.standard_normal(100), rng.standard_normal(100)
    z = np.zeros(100)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    pn, m, v = oracle.adamw_step(p, g, z, z, lr, b1, b2, eps, wd, 1)
    assert np.allclose(m, 0.1 * g, rtol=1e-14) and np.allclose(v, 0.001 * g * g, rtol=1e-12)
    assert np.allclose(pn, p - lr * (g / (np.abs(g) + eps) + wd * p), rtol=1e-12, atol=1e-15)


def test_constant_gradient_keeps_the_corrected_moments_exact():
    # m_t = g (1 - b1^t) and v_t = g^2 (1 - b2^t): each step moves p by
    # lr g / (|g| + eps) (no decay)
    g = np.array([0.5, -2.0, 3e-3, -7.0])
    p = np.array([1.0, 2.0, -3.0, 0.25])
    m = v = np.zeros(4)
    lr, b1, b2, eps = 0.01, 0.9, 0.99, 1e-8
    p0 = p.copy()
    for t in range(1, 51):
        p, m, v = oracle.adamw_step(p, g, m, v, lr, b1, b2, eps, 0.0, t)
    assert np.allclose(m, g * (1 - b1 ** 50), rtol=1e-12)
    assert np.allclose(p, p0 - 50 * lr * g / (np.abs(g) + eps), rtol=1e-10)


def test_pure_weight_decay():
    # zero gradients leave m = v = 0 and shrink p by (1 - lr wd) per step
    p = np.array([1.0, -4.0, 0.5])
    z = np.zeros(3)
    m = v = z
    for t in range(1, 11):
        p, m, v = oracle.adamw_step(p, z, m, v, 0.1, 0.9, 0.999, 1e-8, 0.2, t)
    assert np.allclose(p, np.array([1.0, -4.0, 0.5]) * (1 - 0.02) ** 10, rtol=1e-13)
    assert np.all(m == 0) and np.all(v == 0)


def test_zero_betas_use_the_current_gradient_only():
    rng = np.random.default_rng(1)
    p, g, m, v = (rng.standard_normal(50) for _ in range(4))
    v = np.abs(v)
    pn, mn, vn = oracle.adamw_step(p, g, m, v, 1e-2, 0.0, 0.0, 1e-6, 0.0, 7)
    assert np.array_equal(mn, g) and np.array_equal(vn, g * g)
    assert np.allclose(pn, p - 1e-2 * g / (np.abs(g) + 1e-6), rtol=1e-13)
