"""The 4-bit codebooks the pages compare NF4 with: FP4 and Int4.

The pages state that NF4 has a lower quantization error than Int4 and FP4
and gives higher accuracy than both (deepfa.ir page, "1. 4-bit NormalFloat
(NF4)" feature list and the NF4 efficiency point of its results list); the
glossary page ("Definition" and the results paragraph) says QLoRA with a
plain 4-bit float scored about one point lower than with NF4.  Neither
format is defined there.  Readings (the plainest formats of those names):

  R15 FP4 is E2M1: a sign bit, two exponent bits with bias 1 (exponent
      field 0 is subnormal: 0 or 0.5) and one mantissa bit, so the values
      are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Normalised by the largest (6) and
      sorted ascending into 16 codes; its two zeros are both +0 (codes 7
      and 8), and with ties to the lower index code 8 never occurs.
  R16 Int4 is a two's-complement 4-bit integer k = -8..7 scaled by 1/7, so
      that an absmax-normalised x in [-1, 1] maps to k/7, k = -7..7; the
      code for -8/7 lies outside [-1, 1] and never occurs.

Both are quantized exactly like NF4 (readings R2-R10): blockwise absmax,
nearest level with ties to the lower index, the same 8-bit double
quantization of the block absmaxes.  An all-zero block stores the code of
the level 0 (the lowest such index: 7 for NF4 and FP4, 8 for Int4).
"""

from fractions import Fraction

import numpy as np

from .nf4 import nf4_levels


def e2m1_value(code):
    """The value of a 4-bit E2M1 pattern (sign, exponent[2], mantissa[1])."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def fp4_levels():
    """FP4 (R15): the 16 E2M1 values divided by 6, ascending, RN to fp32."""
    vals = sorted(e2m1_value(c) / 6 for c in range(16))
    return np.array([float(v) for v in vals], dtype=np.float64).astype(np.float32) + np.float32(0.0)


def int4_levels():
    """Int4 (R16): k/7 for k = -8..7, ascending, RN to fp32."""
    return np.array([k / 7.0 for k in range(-8, 8)], dtype=np.float64).astype(np.float32)


CODEBOOKS = {"nf4": nf4_levels, "fp4": fp4_levels, "int4": int4_levels}


def levels(codebook):
    """The 16 fp32 levels of a codebook by name ("nf4", "fp4", "int4")."""
    return CODEBOOKS[codebook]()


def zero_code(lv):
    """The code an all-zero block stores: the lowest index of a zero level."""
    return int(np.flatnonzero(np.asarray(lv) == 0)[0])
