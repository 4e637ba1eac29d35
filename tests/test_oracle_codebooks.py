"""Pins for the oracle's FP4 and Int4 codebooks (CPU only).

Pinned against: the E2M1 value list of the format's definition (sign,
exponent with bias 1, one mantissa bit), exact rational rounding of every
level, brute-force exact nearest-level search on small blocks for every
codebook (ties to the lower index, the zero-block code), and the pages'
claim that NF4 has a lower quantization error than FP4 and Int4.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_quantized_finetuning_nf4_amd import synth


def _rn32(q):
    """Exact round-to-nearest-even of a rational to fp32 (brute force)."""
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return np.float32(min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                                int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)))


def test_e2m1_decoding_matches_the_format():
    # E2M1 magnitudes: exponent field 0 -> 0 and 0.5 (subnormal), then
    # 1, 1.5 / 2, 3 / 4, 6; the sign bit negates
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    for code in range(16):
        sign = -1 if code & 8 else 1
        assert oracle.e2m1_value(code) == sign * mags[code & 7], code


def test_fp4_levels():
    lv = oracle.fp4_levels()
    assert lv.dtype == np.float32 and lv.size == 16
    want = sorted(oracle.e2m1_value(c) / 6 for c in range(16))
    for k in range(16):
        assert lv[k] == _rn32(want[k]), k
    assert lv[0] == -1.0 and lv[15] == 1.0
    assert np.all(np.diff(lv.astype(np.float64)) >= 0)
    # the two zeros are +0 at codes 7 and 8; every other level is distinct
    assert list(np.flatnonzero(lv == 0)) == [7, 8]
    assert not np.signbit(lv[7]) and not np.signbit(lv[8])
    assert np.unique(lv).size == 15
    assert oracle.zero_code(lv) == 7


def test_int4_levels():
    lv = oracle.int4_levels()
    assert lv.dtype == np.float32 and lv.size == 16
    for k in range(16):
        assert lv[k] == _rn32(Fraction(k - 8, 7)), k
    assert np.all(np.diff(lv.astype(np.float64)) > 0)
    assert lv[1] == -1.0 and lv[15] == 1.0 and lv[8] == 0.0
    assert oracle.zero_code(lv) == 8


def _exact_codes(w_bits, lv):
    """Codes by exact rational arithmetic: x = RN32(w / a), nearest level,
    ties to the lower index; an all-zero block gets the first zero level."""
    w = oracle.bf16_bits_to_f64(w_bits)
    out = []
    for b in range(0, w.size, 64):
        blk = [Fraction(float(v)) for v in w[b:b + 64]]
        a = max(abs(v) for v in blk)
        for v in blk:
            if a == 0:
                out.append(int(np.flatnonzero(lv == 0)[0]))
                continue
            x = Fraction(float(_rn32(v / a)))
            d = [abs(x - Fraction(float(l))) for l in lv]
            out.append(d.index(min(d)))
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "int4"])
def test_quantize_codes_brute_force(codebook):
    lv = oracle.codebook_levels(codebook)
    rng = np.random.default_rng(3)
    w = rng.standard_normal(64 * 6) * 0.02
    w[64:128] = 0.0                                        # an all-zero block
    w[128:192] = np.round(w[128:192] * 500) / 500          # ties on coarse values
    # values landing on the midpoints between levels: w = a * mid
    a = 0.05
    w[192] = a
    mids = (lv[:-1].astype(np.float64) + lv[1:].astype(np.float64)) / 2
    w[193:193 + 15] = a * mids
    bits = synth.to_bf16_bits(w)
    codes, _, _ = oracle.quantize(bits, codebook)
    got = np.stack([codes & 15, codes >> 4], axis=1).ravel()[:bits.size]
    assert np.array_equal(got, _exact_codes(bits, lv))


@pytest.mark.parametrize("codebook", ["fp4", "int4"])
def test_dequant_round_trip(codebook):
    # a block holding exactly a * level for each level (a a power of two,
    # group scale a) comes back unchanged
    lv = oracle.codebook_levels(codebook)
    vals = [float(v) for v in lv if -1 <= v <= 1]
    w = np.zeros(64, dtype=np.float64)
    w[:len(vals)] = np.array(vals) * 0.25
    bits = synth.to_bf16_bits(w)
    exact = oracle.bf16_bits_to_f64(bits)
    c, aq, s2 = oracle.quantize(bits, codebook)
    back = oracle.bf16_bits_to_f64(oracle.dequant(c, aq, s2, bits.size, codebook))
    # bf16 holds levels like 1/3 only to 8 bits, so compare with the bf16 of
    # the dequantized value of the level the weight quantizes to
    codes = np.stack([c & 15, c >> 4], axis=1).ravel()[:bits.size]
    want = oracle.bf16_bits_to_f64(synth.to_bf16_bits(lv[codes].astype(np.float64) * 0.25))
    assert np.array_equal(back, want)
    assert np.max(np.abs(back - exact)) <= 0.25 * 2 ** -7


def test_nf4_has_the_lowest_quantization_error():
    # the pages: NF4 has lower quantization error than Int4 and FP4; on
    # normally distributed weights, through the whole storage path
    rng = np.random.default_rng(1)
    bits = synth.to_bf16_bits(rng.standard_normal(1 << 16) * 0.02)
    w = oracle.bf16_bits_to_f64(bits)
    err = {}
    for cb in ("nf4", "fp4", "int4"):
        c, a, s = oracle.quantize(bits, cb)
        d = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, bits.size, cb))
        err[cb] = np.sqrt(np.mean((d - w) ** 2))
    assert err["nf4"] < err["fp4"] and err["nf4"] < err["int4"], err
