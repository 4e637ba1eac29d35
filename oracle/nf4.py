"""The two codebooks of the method, computed from their definitions.

NF4 (deepfa.ir page, section "1. 4-bit NormalFloat (NF4)"; glossary page,
"Definition"; insights4ai page, feature list item (a)): a 4-bit data type
built for normally distributed weights, in which each bucket receives an
equal share of the values.  The pages give no formula.

Reading R1 (the plainest construction meeting every stated property:
16 levels, normal quantiles, equal probability per bucket, normalised to
[-1, 1], an exact zero, strictly monotone):

  * delta = 929/960, the mean of (1 - 1/30) and (1 - 1/32), keeps the
    inverse normal CDF finite at the extreme level;
  * 8 positive levels  Phi^-1(p) at p = delta + (1/2 - delta) * j/8, j = 0..7;
  * 7 negative levels -Phi^-1(p) at p = delta + (1/2 - delta) * j/7, j = 0..6;
  * the level 0;
  * divide all by Phi^-1(delta), sort ascending, round each to fp32.

Phi^-1 is Python's ``statistics.NormalDist().inv_cdf`` (Wichura's AS241
algorithm, accurate to about 1e-16).

Second-level 8-bit codebook (reading R9; the glossary page "Definition" and
the deepfa.ir page "2. Double Quantization" only say that the scaling
constants are themselves quantized): an unsigned linear code on [0, 1],
Q8[k] = RN32(k / 255), k = 0..255.
"""

from fractions import Fraction
from statistics import NormalDist

import numpy as np

NF4_OFFSET = Fraction(929, 960)


def nf4_levels_fp64(inv_cdf=None):
    """NF4 levels in fp64, ascending (index 0 = -1, 7 = 0, 15 = +1).

    ``inv_cdf`` may be passed to rebuild the table with another inverse
    normal CDF (the tests use an independent one as a cross-check).
    """
    if inv_cdf is None:
        inv_cdf = NormalDist().inv_cdf
    delta = float(NF4_OFFSET)
    z = inv_cdf(delta)
    pos = [inv_cdf(delta + (0.5 - delta) * j / 8) / z for j in range(8)]
    neg = [-inv_cdf(delta + (0.5 - delta) * j / 7) / z for j in range(7)]
    levels = sorted(pos + neg + [0.0])
    return np.array(levels, dtype=np.float64)


def nf4_levels(inv_cdf=None):
    """NF4 levels rounded to fp32 (round to nearest even), ascending."""
    return nf4_levels_fp64(inv_cdf).astype(np.float32)


def q8_levels():
    """Second-level codebook Q8[k] = RN32(k/255), k = 0..255.

    k/255 is formed in fp64 and then rounded to fp32; for a quotient of two
    small integers this double rounding equals direct rounding to fp32
    (the test suite checks every entry against exact rational rounding).
    """
    return (np.arange(256, dtype=np.float64) / 255.0).astype(np.float32)
