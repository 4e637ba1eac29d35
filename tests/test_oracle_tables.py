"""Pins for the oracle's codebooks and bf16 conversion (CPU only).

The NF4 table is pinned by its defining properties (16 levels, exact zero,
-1 and +1 at the ends, strictly increasing, equal probability mass between
levels on each side of zero) and by rebuilding it with two independent
inverse normal CDFs (mpmath at 50 digits, scipy's ndtri); the Q8 table by
exact rational rounding; the bf16 cast by torch's own CPU cast.
"""

import json
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch
from scipy.special import ndtri

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _mp_inv_cdf(p):
    mpmath.mp.dps = 50
    return float(mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1))


def test_nf4_table_shape_and_invariants():
    L = oracle.nf4_levels()
    fig = json.load(open(GOLDEN))
    assert L.dtype == np.float32 and L.size == fig["nf4_levels"]["value"]
    assert L[0] == -1.0 and L[15] == 1.0
    assert L[7] == 0.0 and not np.signbit(L[7])
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    # 7 negative levels, zero, 8 positive levels
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8


def test_nf4_table_independent_inverse_cdfs_agree_bitwise():
    ref = oracle.nf4_levels().view(np.uint32)
    mp = oracle.nf4_levels(inv_cdf=_mp_inv_cdf).view(np.uint32)
    sp = oracle.nf4_levels(inv_cdf=lambda p: float(ndtri(p))).view(np.uint32)
    assert np.array_equal(ref, mp)
    assert np.array_equal(ref, sp)
    # and each fp64 level sits far from an fp32 rounding tie, so any inverse
    # CDF accurate to ~1e-12 reproduces the fp32 table
    L64 = oracle.nf4_levels_fp64(inv_cdf=_mp_inv_cdf)
    for v in L64:
        f = np.float32(v)
        if v == 0 or abs(v) == 1:
            continue
        ulp = abs(np.float64(np.nextafter(f, np.float32(np.inf))) - np.float64(f))
        frac = abs(v - np.float64(f)) / ulp
        assert frac < 0.49, v


def test_nf4_equal_probability_mass_per_side():
    # equal-occupancy buckets for N(0,1) data: Phi(L * z) is evenly spaced on
    # each side of zero (deepfa.ir blog, "1. 4-bit NormalFloat (NF4)")
    mpmath.mp.dps = 50
    z = _mp_inv_cdf(float(oracle.NF4_OFFSET))
    L = oracle.nf4_levels_fp64(inv_cdf=_mp_inv_cdf)
    p = np.array([float(mpmath.ncdf(v * z)) for v in L])
    neg_steps = np.diff(p[:8])           # -1 .. 0 : 7 steps
    pos_steps = np.diff(p[7:])           #  0 .. 1 : 8 steps
    assert np.allclose(neg_steps, neg_steps[0], rtol=0, atol=1e-13)
    assert np.allclose(pos_steps, pos_steps[0], rtol=0, atol=1e-13)
    delta = float(oracle.NF4_OFFSET)
    assert abs(neg_steps[0] - (delta - 0.5) / 7) < 1e-13
    assert abs(pos_steps[0] - (delta - 0.5) / 8) < 1e-13
    assert abs(p[15] - delta) < 1e-13 and abs(p[0] - (1 - delta)) < 1e-13


def _round_fraction_to_f32(q):
    """Exact round-to-nearest-even of a rational to fp32 (brute force)."""
    f = np.float32(float(q))                       # within one ulp
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, dtype=np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_q8_table_exact_rational_rounding():
    Q = oracle.q8_levels()
    assert Q.dtype == np.float32 and Q.size == 256
    for k in range(256):
        assert Q[k] == _round_fraction_to_f32(Fraction(k, 255)), k
    assert Q[0] == 0.0 and Q[255] == 1.0
    assert np.all(np.diff(Q.astype(np.float64)) > 0)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),       # fp32 denormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38], dtype=np.float32),
    ])
    # exact ties: low 16 bits = 0x8000 with even and odd kept parts
    ties = (rng.integers(0, 2**15, 5000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    ours = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_widening_round_trip():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(b)
    fin = np.isfinite(f)
    assert np.array_equal(oracle.f32_to_bf16_bits(f[fin]), b[fin])
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f[fin].view(np.uint32), t[fin].view(np.uint32))
