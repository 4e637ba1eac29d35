"""CPU oracle for the NF4 + double-quantization + LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct reference that the GPU library is checked against.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  The GPU library never calls it and shares no
code, table or helper with it.

Sources (the QLoRA pages):
  * "QLoRA" glossary page (mangrove.ai), section "Definition": frozen 4-bit
    weights, converted back to BFloat16 each time a layer is used, LoRA
    matrices trained in 16-bit, weight gradients only for the LoRA matrices,
    double quantization saving about 0.37 bit per parameter.
  * "QLoRA: Fine-Tuning 65-Billion Parameter Models on a Single Consumer GPU"
    (deepfa.ir), sections "LoRA: Prerequisite", "1. 4-bit NormalFloat (NF4)",
    "2. Double Quantization" and "QLoRA's Working Process".

Where those pages leave a step open, the reading taken is stated in the
docstring of the function that implements it (readings R1-R20).

Every function here is pinned by a test in ``tests/test_oracle_*.py``
against something other than itself (closed forms, exact rational
arithmetic, brute force, invariants); none is "parity unpinned".
"""

from .nf4 import nf4_levels, nf4_levels_fp64, q8_levels, NF4_OFFSET
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32, bf16_bits_to_f64
from .quant import (nf4_encode, q8_encode, quantize, dequant, storage_sizes,
                    BLOCKSIZE, GROUP_BLOCKS)
from .linear import linear_fwd, linear_bwd, adapter_grads, gemv, lora_scale
from .codebooks import fp4_levels, int4_levels, e2m1_value, zero_code, CODEBOOKS
from .codebooks import levels as codebook_levels
from .optim import adamw_step
from .group import group_fwd, group_bwd
from .secondlevel import e4m3_value, fp8_levels, FORMATS as ABSMAX_FORMATS
from .secondlevel import levels as absmax_levels

__all__ = [
    "nf4_levels", "nf4_levels_fp64", "q8_levels", "NF4_OFFSET",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "nf4_encode", "q8_encode", "quantize", "dequant", "storage_sizes",
    "BLOCKSIZE", "GROUP_BLOCKS",
    "linear_fwd", "linear_bwd", "gemv", "lora_scale",
    "fp4_levels", "int4_levels", "e2m1_value", "zero_code", "CODEBOOKS", "codebook_levels",
    "adamw_step", "group_fwd", "group_bwd", "e4m3_value", "fp8_levels", "ABSMAX_FORMATS", "absmax_levels",
]
