"""bfloat16 <-> fp32 by explicit bit arithmetic.

The compute dtype of the layer is BFloat16 (glossary page "Definition": the
4-bit weights are converted back to BFloat16 each time a layer is used).
bfloat16 is the top 16 bits of an IEEE fp32; the conversion from fp32 rounds
to nearest, ties to even.  NaN inputs are out of scope (weights and
activations are finite).
"""

import numpy as np


def f32_to_bf16_bits(x):
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lower = u & np.uint64(0xFFFF)
    upper = u >> np.uint64(16)
    odd = upper & np.uint64(1)
    # round up when the discarded half is above one half, or exactly one
    # half and the kept part is odd
    up = (lower > np.uint64(0x8000)) | ((lower == np.uint64(0x8000)) & (odd == np.uint64(1)))
    out = upper + up.astype(np.uint64)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bfloat16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b):
    """Exact widening of bfloat16 bit patterns to fp64."""
    return bf16_bits_to_f32(b).astype(np.float64)
