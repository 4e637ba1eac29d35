"""Blockwise NF4 quantization with double-quantized block constants.

What the pages fix: the frozen pretrained weights are stored as 4-bit NF4
numbers (glossary page "Definition"; deepfa.ir "1. 4-bit NormalFloat"),
quantization needs constants that scale the quantized values, usually kept
in fp32, and double quantization quantizes those constants a second time
(deepfa.ir "2. Double Quantization"; glossary "Definition"); the weights are
converted back to BFloat16 each time the layer is used.

Readings for what the pages leave open (the geometry comes from the task's
problem statement, the rest is the plainest reading):

  R2  normalisation x = RN32(w / a_b), a correctly rounded fp32 division.
  R3  nearest level, ties to the lower index.
  R4  ascending level indices (0 = -1, 7 = 0, 15 = +1).
  R5  a block is 64 consecutive elements of the row-major weight; a_b is
      the largest |w| in it (exact, fp32).
  R6  an all-zero block stores code 7 (the exact zero) everywhere.
  R7  a short last block / last group covers the elements present; an odd
      element count leaves the high nibble of the last byte zero.
  R8  element 2j goes to the low nibble of byte j, element 2j+1 to the high.
  R9  second level: groups of 256 blocks, s2 = max a_b of the group (fp32),
      y = RN32(a_b / s2), stored as the index of the nearest Q8 level
      (ties to the lower index); no mean subtraction.
  R10 an all-zero group stores s2 = 0 and codes 0.

Dequantization (the BFloat16 value used by the layer):
  t  = RN32(Q8[q_b] * s2_g)
  w' = RN32(L[c] * t)
  out = RNE_bf16(w')
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from .nf4 import nf4_levels, q8_levels
from .codebooks import levels as codebook_levels, zero_code
from .secondlevel import levels as absmax_levels

BLOCKSIZE = 64
GROUP_BLOCKS = 256
_CHUNK = 1 << 20


def _nearest_index(values, levels):
    """Index of the nearest level for each value; ties go to the lower index.

    Distances are formed in fp64, where the difference of two fp32 numbers
    of magnitude <= 1 is exact; np.argmin returns the first minimum, which is
    the lower index on a tie.
    """
    values = np.asarray(values, dtype=np.float32).ravel()
    lv = np.asarray(levels, dtype=np.float64)
    out = np.empty(values.size, dtype=np.uint8)
    for s in range(0, values.size, _CHUNK):
        v = values[s:s + _CHUNK].astype(np.float64)
        d = np.abs(v[:, None] - lv[None, :])
        out[s:s + _CHUNK] = np.argmin(d, axis=1).astype(np.uint8)
    return out


def nf4_encode(x):
    """NF4 code of normalised fp32 values x in [-1, 1] (readings R3, R4)."""
    return _nearest_index(x, nf4_levels())


def q8_encode(y):
    """8-bit second-level code of fp32 values y in [0, 1] (reading R9)."""
    return _nearest_index(y, q8_levels())


def storage_sizes(numel):
    """Bytes of (codes, absmax codes, group scales) for `numel` weights."""
    nb = -(-numel // BLOCKSIZE)
    ng = -(-nb // GROUP_BLOCKS)
    return (numel + 1) // 2, nb, 4 * ng


def quantize(w_bits, codebook="nf4", absmax_format="linear"):
    """Quantize bf16 weights (uint16 bit patterns, row-major, any shape).

    Returns (codes uint8 [ceil(n/2)], absmax_q uint8 [nb], s2 float32 [ng]).
    ``codebook`` selects the 4-bit levels: "nf4" (the method's), or "fp4"
    and "int4" (the formats the pages compare it with; readings R15, R16 in
    codebooks.py), all quantized the same way.  ``absmax_format`` selects the
    second-level code: "linear" (R9) or "fp8" (R19, secondlevel.py).
    """
    lv = codebook_levels(codebook)
    w = bf16_bits_to_f32(np.asarray(w_bits).ravel())
    n = w.size
    nb = -(-n // BLOCKSIZE)
    ng = -(-nb // GROUP_BLOCKS)

    # first level: block absmax (zero padding does not change a max of |w|)
    padded = np.zeros(nb * BLOCKSIZE, dtype=np.float32)
    padded[:n] = w
    blocks = padded.reshape(nb, BLOCKSIZE)
    absmax = np.max(np.abs(blocks), axis=1)                      # fp32, exact

    # normalise and encode; blocks with absmax 0 keep the code of the level 0
    # (7 for NF4: R6)
    codes_full = np.full(nb * BLOCKSIZE, zero_code(lv), dtype=np.uint8)
    nz = absmax > 0
    if np.any(nz):
        x = (blocks[nz] / absmax[nz, None]).astype(np.float32)    # IEEE fp32 division
        codes_full.reshape(nb, BLOCKSIZE)[nz] = _nearest_index(x, lv).reshape(-1, BLOCKSIZE)
    codes_el = codes_full[:n]

    # pack two codes per byte, element 2j in the low nibble (R8)
    if n % 2:
        codes_el = np.concatenate([codes_el, np.zeros(1, dtype=np.uint8)])
    packed = (codes_el[0::2] | (codes_el[1::2] << 4)).astype(np.uint8)

    # second level: per group of 256 blocks (R9, R10)
    apad = np.zeros(ng * GROUP_BLOCKS, dtype=np.float32)
    apad[:nb] = absmax
    s2 = np.max(apad.reshape(ng, GROUP_BLOCKS), axis=1).astype(np.float32)
    s2_per_block = np.repeat(s2, GROUP_BLOCKS)[:nb]
    absmax_q = np.zeros(nb, dtype=np.uint8)
    gz = s2_per_block > 0
    if np.any(gz):
        y = (absmax[gz] / s2_per_block[gz]).astype(np.float32)
        absmax_q[gz] = _nearest_index(y, absmax_levels(absmax_format))
    return packed, absmax_q, s2


def dequant(codes, absmax_q, s2, numel, codebook="nf4", absmax_format="linear"):
    """Dequantize to bf16 bit patterns (uint16, flat, `numel` elements)."""
    codes = np.asarray(codes, dtype=np.uint8)
    el = np.empty(2 * codes.size, dtype=np.uint8)
    el[0::2] = codes & 0x0F
    el[1::2] = codes >> 4
    el = el[:numel]
    blk = np.arange(numel) // BLOCKSIZE
    grp = blk // GROUP_BLOCKS
    q8 = absmax_levels(absmax_format)
    lv = codebook_levels(codebook)
    t = (q8[np.asarray(absmax_q)[blk]] * np.asarray(s2, dtype=np.float32)[grp]).astype(np.float32)
    w = (lv[el] * t).astype(np.float32)
    return f32_to_bf16_bits(w)
