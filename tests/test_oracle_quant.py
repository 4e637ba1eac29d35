"""Pins for the oracle's quantize / dequantize (CPU only).

Pinned against: exact rational nearest-level search (brute force), hand-made
blocks with known codes, the double-quantization closed form and the
memory figures printed on the pages (tests/golden/pages_figures.json),
the quantization error bound implied by the level spacing, the round-trip
identity, zero-padding invariance of the tail rule, and the pages' claim
that NF4 has lower quantization error than Int4 on normal data.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_nf4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _exact_nearest(x, levels):
    fx = Fraction(float(x))
    d = [abs(fx - Fraction(float(v))) for v in levels]
    m = min(d)
    return d.index(m)        # first minimum = lower index on a tie


def _neighbourhood(v, n):
    f = np.float32(v)
    out = [f]
    lo = hi = f
    for _ in range(n):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return out


def test_nf4_encode_matches_exact_argmin_near_every_midpoint():
    L = oracle.nf4_levels()
    xs = []
    for k in range(15):
        mid = (np.float64(L[k]) + np.float64(L[k + 1])) / 2
        xs += _neighbourhood(mid, 8)
    rng = np.random.default_rng(2)
    xs += list(rng.uniform(-1, 1, 3000).astype(np.float32))
    xs += [np.float32(v) for v in L] + [np.float32(-1.0), np.float32(1.0), np.float32(0.0)]
    xs = np.array(xs, dtype=np.float32)
    got = oracle.nf4_encode(xs)
    want = np.array([_exact_nearest(x, L) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_nf4_exact_midpoints_go_to_lower_index():
    L = oracle.nf4_levels()
    exact = 0
    for k in range(15):
        mid = (np.float64(L[k]) + np.float64(L[k + 1])) / 2
        if np.float64(np.float32(mid)) == mid:
            exact += 1
            assert oracle.nf4_encode(np.array([mid], dtype=np.float32))[0] == k
    assert exact >= 1          # at least one level pair has an fp32 midpoint


def test_q8_encode_matches_exact_argmin():
    Q = oracle.q8_levels()
    xs = []
    for k in range(0, 255, 7):
        mid = (np.float64(Q[k]) + np.float64(Q[k + 1])) / 2
        xs += _neighbourhood(mid, 3)
    rng = np.random.default_rng(3)
    xs += list(rng.uniform(0, 1, 500).astype(np.float32))
    xs = np.array(xs, dtype=np.float32)
    got = oracle.q8_encode(xs)
    want = np.array([_exact_nearest(x, Q) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def _bits(v):
    return synth.to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_hand_block_codes_and_packing():
    w = np.zeros(64, dtype=np.float32)
    w[0], w[1], w[2], w[3] = 0.5, -0.5, 0.0, 0.25      # a = 0.5, x = 1, -1, 0, 0.5
    codes, aq, s2 = oracle.quantize(_bits(w))
    el = np.empty(64, dtype=np.uint8)
    el[0::2], el[1::2] = codes & 15, codes >> 4
    L = oracle.nf4_levels()
    assert el[0] == 15 and el[1] == 0 and el[2] == 7
    assert el[3] == np.argmin(np.abs(L.astype(np.float64) - 0.5))    # 0.5 -> level 12 (0.4407)
    assert el[3] == 12
    assert codes[0] == (15 | (0 << 4)) and codes[1] == (7 | (12 << 4))
    assert np.all(el[4:64] == 7)
    # one block, one group: s2 = a and the block's own code is 255 (Q8 = 1.0)
    assert s2.shape == (1,) and s2[0] == np.float32(0.5) and aq[0] == 255


def test_zero_block_and_zero_group():
    w = np.zeros(64 * 300, dtype=np.float32)
    w[64 * 256 + 5] = 1.0                 # only the second group has a non-zero block
    codes, aq, s2 = oracle.quantize(_bits(w))
    assert s2[0] == 0 and np.all(aq[:256] == 0)
    assert np.all(codes[:64 * 256 // 2] == 0x77)
    assert s2[1] == 1.0 and aq[256] == 255
    deq = oracle.bf16_bits_to_f32(oracle.dequant(codes, aq, s2, w.size))
    assert np.all(deq[:64 * 256] == 0)
    assert deq[64 * 256 + 5] == 1.0


def test_tail_equals_zero_padding_and_odd_count():
    rng = np.random.default_rng(4)
    n = 64 * 257 + 37                     # ragged block and ragged group
    wb = _bits(rng.standard_normal(n) * 0.02)
    codes, aq, s2 = oracle.quantize(wb)
    pad = np.concatenate([wb, np.zeros(64 * 258 - n, dtype=np.uint16)])
    pc, paq, ps2 = oracle.quantize(pad)
    nb = -(-n // 64)
    assert codes.size == (n + 1) // 2 and aq.size == nb and s2.size == 2
    assert np.array_equal(codes[:-1], pc[:codes.size - 1])
    # odd count: last byte holds the last element in its low nibble only
    assert codes[-1] >> 4 == 0 and (codes[-1] & 15) == (pc[codes.size - 1] & 15)
    assert np.array_equal(aq, paq[:nb]) and np.array_equal(s2, ps2)


def test_storage_and_double_quantization_closed_form():
    fig = json.load(open(GOLDEN))
    n = 8192 * 8192
    cb, ab, sb = oracle.storage_sizes(n)
    bits = 8 * (cb + ab + sb) / n
    assert bits == 4 + 8 / 64 + 32 / (64 * 256)
    bits_fp32_constants = 4 + 32 / 64
    saving = bits_fp32_constants - bits
    assert saving == 32 / 64 - (8 / 64 + 32 / (64 * 256))      # 0.373046875
    f = fig["dq_saving_bits_per_param"]
    assert abs(saving - f["value"]) <= f["tolerance"]
    g = fig["dq_saving_gb_at_65b"]
    assert abs(saving * g["params"] / 8 / 1e9 - g["value"]) <= g["tolerance"]


def test_65b_nf4_footprint_under_48gb():
    fig = json.load(open(GOLDEN))
    total = 0
    for _, N, K in synth.LAYER_SETS["llama65b"]["linears"]:
        total += sum(oracle.storage_sizes(N * K))
    total *= synth.DECODE_LAYERS
    assert 30e9 < total < fig["qlora_65b_memory_gb_upper"]["value"] * 1e9


def test_dequant_error_bound_and_round_trip():
    d = synth.small_numpy(0)
    W = d["W"]
    codes, aq, s2 = oracle.quantize(W)
    deq_bits = oracle.dequant(codes, aq, s2, W.size)
    w = oracle.bf16_bits_to_f64(W).ravel()
    dq = oracle.bf16_bits_to_f64(deq_bits)
    L = oracle.nf4_levels().astype(np.float64)
    a = np.max(np.abs(w.reshape(-1, 64)), axis=1)
    half_gap = np.max(np.diff(L)) / 2                       # largest half-gap, 0.1519
    el = np.empty(2 * codes.size, dtype=np.uint8)
    el[0::2], el[1::2] = codes & 15, codes >> 4
    s2b = np.repeat(s2.astype(np.float64), 256)[: a.size]
    bound = (half_gap * np.repeat(a, 64) + np.abs(L[el]) * np.repeat(s2b / 510 + 2.0**-23 * s2b, 64)
             + 2.0**-8 * np.abs(dq) + 1e-12)
    assert np.all(np.abs(w - dq) <= bound)
    # every group's largest block reconstructs its absmax exactly (code 255)
    assert np.all(aq.reshape(-1, 256).max(axis=1) == 255)
    # quantize(dequant(quantize(W))) reproduces the NF4 codes exactly
    c2, aq2, s22 = oracle.quantize(deq_bits)
    assert np.array_equal(c2, codes)
    assert np.max(np.abs(aq2.astype(int) - aq.astype(int))) <= 1


def test_nf4_beats_int4_on_normal_blocks():
    # deepfa.ir blog, "1. 4-bit NormalFloat (NF4)": lower quantization error
    # than Int4 on normally distributed weights
    rng = np.random.default_rng(5)
    w = (rng.standard_normal(64 * 20000) * 0.02).astype(np.float32)
    wb = synth.to_bf16_bits(w)
    codes, aq, s2 = oracle.quantize(wb)
    wf = oracle.bf16_bits_to_f64(wb)
    nf4 = oracle.bf16_bits_to_f64(oracle.dequant(codes, aq, s2, wf.size))
    blocks = wf.reshape(-1, 64)
    a = np.max(np.abs(blocks), axis=1, keepdims=True)
    int4 = np.round(blocks / a * 7) / 7 * a                   # symmetric absmax Int4
    mse_nf4 = np.mean((wf - nf4) ** 2)
    mse_int4 = np.mean((blocks - int4) ** 2)
    assert mse_nf4 < mse_int4
