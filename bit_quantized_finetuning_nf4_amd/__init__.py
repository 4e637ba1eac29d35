"""MI355X-native QLoRA hot path: NF4 + double-quantized frozen linear layer with
a bf16 LoRA adapter (forward, backward, batch-1 decode).

The compute runs in libqlora.so (hand-written gfx950 HIP kernels behind a C
ABI, include/qlora.h); this package is its thin Python binding.  The library
is loaded on the first call and a missing build is an error.
"""

from .ops import (GemvJob, QuantizedWeight, dequant, gemv, linear_bwd, linear_fwd, nf4_levels,
                  quantize, sizes, workspace, workspace_bytes)

__all__ = ["GemvJob", "QuantizedWeight", "dequant", "gemv", "linear_bwd", "linear_fwd", "nf4_levels",
           "quantize", "sizes", "workspace", "workspace_bytes"]
__version__ = "0.1.0"
