"""Second-level formats for the double-quantized block constants.

The pages say only that double quantization quantizes the quantization
constants a second time, to about 0.37 bit per parameter saved (glossary
page "Definition"; deepfa.ir "2. Double Quantization"); they name no format.
Two 8-bit codes are built, both applied to y = RN32(a_b / s2) in [0, 1]
(s2 = the largest block absmax of the group of 256 blocks) and decoded as
t = RN32(Q[q] * s2):

  "linear" (reading R9): Q[k] = RN32(k / 255), k = 0..255: uniform steps of
           s2 / 255, so a block whose absmax is below s2 / 510 is stored as 0;
  "fp8"    (reading R19): FP8 E4M3, read as the common 8-bit float with a
           sign bit (always 0 here), four exponent bits with bias 7 (field 0:
           subnormal) and three mantissa bits, largest finite value 448 at
           code 0x7E (0x7F is not a number and is never produced).
           Q[k] = RN32(e4m3(k) / 448), k = 0..126: relative steps of 1/8 to
           1/16 over [2^-15, 1], so small block constants keep their
           relative precision.

Both take the nearest level with ties to the lower index, and both decode the
group's largest block exactly (Q = 1).
"""

from fractions import Fraction

import numpy as np

from .nf4 import q8_levels

FORMATS = ("linear", "fp8")
FP8_MAX_CODE = 126


def e4m3_value(k):
    """Exact value of the non-negative FP8 E4M3 bit pattern k (0..126)."""
    e, m = (k >> 3) & 15, k & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 2 ** 6)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _round_f32(x):
    """Correctly rounded fp32 of an exact rational x > 0 (round to nearest even)."""
    lo = np.float32(float(x))
    # float(x) is correctly rounded to fp64; step to the fp32 neighbours and
    # pick the nearest exactly
    cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def fp8_levels():
    """Q[k] = RN32(e4m3(k) / 448), k = 0..126, ascending (reading R19)."""
    return np.array([_round_f32(e4m3_value(k) / 448) for k in range(FP8_MAX_CODE + 1)], dtype=np.float32)


def levels(fmt):
    if fmt == "linear":
        return q8_levels()
    if fmt == "fp8":
        return fp8_levels()
    raise ValueError(f"unknown second-level format {fmt!r}; one of {FORMATS}")
