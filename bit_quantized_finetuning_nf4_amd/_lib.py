"""ctypes view of libqlora.so (include/qlora.h).

The library is loaded on first use from this package directory.  There is no
fallback: a missing library is an error.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_OK = 0
QLORA_OP_FWD, QLORA_OP_BWD, QLORA_OP_GEMV, QLORA_OP_LORA = 0, 1, 2, 3
QLORA_OP_FWD_FUSED, QLORA_OP_BWD_FUSED = 4, 5
QLORA_OP_GROUP_FWD, QLORA_OP_GROUP_BWD, QLORA_OP_GROUP_LORA, QLORA_OP_BF16_DX = 6, 7, 8, 9

STATUS_NAMES = {
    0: "QLORA_OK", 1: "QLORA_E_NULL", 2: "QLORA_E_ALIGN", 3: "QLORA_E_SHAPE",
    4: "QLORA_E_UNSUPPORTED", 5: "QLORA_E_WORKSPACE", 6: "QLORA_E_HIP",
    7: "QLORA_E_FORMAT", 8: "QLORA_E_TABLE",
}
QLORA_E_FORMAT, QLORA_E_TABLE = 7, 8
QTENSOR_HEADER_BYTES = 64

# every function include/qlora.h declares
EXPORTS = [
    "qlora_status_str", "qlora_last_hip_error", "qlora_version", "qlora_nf4_levels",
    "qlora_sizes", "qlora_workspace_bytes", "qlora_quantize", "qlora_dequant",
    "qlora_codebook_levels", "qlora_adamw",
    "qlora_linear_fwd", "qlora_linear_bwd", "qlora_gemv", "qlora_gemv_prepare", "qlora_gemv_run",
    "qlora_lora_down", "qlora_lora_dy_b", "qlora_lora_grads", "qlora_nf4_fwd", "qlora_nf4_dx",
    "qlora_linear_fwd_noalloc", "qlora_bf16_fwd", "qlora_dequant_t", "qlora_bf16_dx",
    "qlora_paged_layout_of", "qlora_paged_adamw", "qlora_group_fwd", "qlora_group_bwd",
    "qlora_group_dequant", "qlora_group_dequant_t", "qlora_bf16_group_fwd", "qlora_bf16_group_dx",
    "qlora_group_lora_dy_b", "qlora_group_lora_grads",
    "qlora_level_table_id", "qlora_qtensor_header_write", "qlora_qtensor_header_read",
]
QLORA_PAGED_LOAD, QLORA_PAGED_STORE = 1, 2

# QLORA_STATIC_SCRATCH_BYTES: scratch array of qlora_linear_fwd_noalloc per device
STATIC_SCRATCH_BYTES = 32 << 20


class Nf4WeightDesc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("group_blocks", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("group_scale", ctypes.c_void_p),
        ("codebook", ctypes.c_int32),
        ("absmax_format", ctypes.c_int32),
    ]


class GemvJobDesc(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.POINTER(Nf4WeightDesc)),
        ("x", ctypes.c_void_p),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("r", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("y", ctypes.c_void_p),
        ("m", ctypes.c_int32),
    ]


class GemvPlanDesc(ctypes.Structure):
    """qlora_gemv_plan: filled by qlora_gemv_prepare, read by qlora_gemv_run."""
    _fields_ = [("priv", ctypes.c_uint64 * 16)]


class PagedTensorDesc(ctypes.Structure):
    _fields_ = [
        ("p", ctypes.c_void_p),
        ("p_bf16", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("m", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


class PagedLayoutDesc(ctypes.Structure):
    _fields_ = [
        ("resident", ctypes.c_int32),
        ("resident_bytes", ctypes.c_size_t),
        ("chunk", ctypes.c_size_t),
        ("staging_bytes", ctypes.c_size_t),
    ]


class QloraError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        msg = STATUS_NAMES.get(status, str(status))
        try:
            msg = lib().qlora_status_str(status).decode()
            if status == 6:
                msg += f" (hipError {lib().qlora_last_hip_error()})"
        except Exception:  # pragma: no cover
            pass
        super().__init__(f"{what}: {msg}")


_lib = None


def lib():
    """Load libqlora.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m bit_quantized_finetuning_nf4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    W = ctypes.POINTER(Nf4WeightDesc)
    L.qlora_status_str.restype = ctypes.c_char_p
    L.qlora_status_str.argtypes = [ctypes.c_int]
    L.qlora_last_hip_error.restype = ctypes.c_int
    L.qlora_last_hip_error.argtypes = []
    L.qlora_version.restype = ctypes.c_char_p
    L.qlora_version.argtypes = []
    L.qlora_nf4_levels.restype = None
    L.qlora_nf4_levels.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.qlora_sizes.restype = ctypes.c_int
    L.qlora_sizes.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.qlora_workspace_bytes.restype = sz
    L.qlora_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i32, i32]
    L.qlora_quantize.restype = ctypes.c_int
    L.qlora_quantize.argtypes = [vp, W, vp]
    L.qlora_dequant.restype = ctypes.c_int
    L.qlora_dequant.argtypes = [W, vp, vp]
    L.qlora_dequant_t.restype = ctypes.c_int
    L.qlora_dequant_t.argtypes = [W, vp, vp]
    L.qlora_paged_layout_of.restype = ctypes.c_int
    L.qlora_paged_layout_of.argtypes = [ctypes.POINTER(PagedTensorDesc), i32, sz, ctypes.POINTER(PagedLayoutDesc)]
    L.qlora_paged_adamw.restype = ctypes.c_int
    L.qlora_paged_adamw.argtypes = [ctypes.POINTER(PagedTensorDesc), i32, vp, sz, f32, f32, f32, f32, f32, i32, i32,
                                    vp, vp]
    L.qlora_codebook_levels.restype = ctypes.c_int
    L.qlora_codebook_levels.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    L.qlora_adamw.restype = ctypes.c_int
    L.qlora_adamw.argtypes = [vp, vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i32, vp]
    L.qlora_linear_fwd.restype = ctypes.c_int
    L.qlora_linear_fwd.argtypes = [W, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    L.qlora_linear_fwd_noalloc.argtypes = [W, vp, i64, vp, vp, i32, f32, vp, vp, vp]
    L.qlora_linear_bwd.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [W, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.qlora_gemv.restype = ctypes.c_int
    L.qlora_gemv.argtypes = [ctypes.POINTER(GemvJobDesc), i32, vp, sz, vp]
    L.qlora_gemv_prepare.restype = ctypes.c_int
    L.qlora_gemv_prepare.argtypes = [ctypes.POINTER(GemvJobDesc), i32, vp, sz, ctypes.POINTER(GemvPlanDesc), vp]
    L.qlora_gemv_run.restype = ctypes.c_int
    L.qlora_gemv_run.argtypes = [ctypes.POINTER(GemvPlanDesc), vp]
    L.qlora_lora_down.restype = ctypes.c_int
    L.qlora_lora_down.argtypes = [vp, vp, i64, i64, i32, vp, vp, sz, vp]
    L.qlora_lora_dy_b.restype = ctypes.c_int
    L.qlora_lora_dy_b.argtypes = [vp, vp, i64, i64, i32, vp, vp, sz, vp]
    L.qlora_lora_grads.restype = ctypes.c_int
    L.qlora_lora_grads.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, f32, vp, vp, vp, sz, vp]
    L.qlora_nf4_fwd.restype = ctypes.c_int
    L.qlora_nf4_fwd.argtypes = [W, vp, i64, vp, vp, i32, f32, vp, vp]
    L.qlora_bf16_fwd.restype = ctypes.c_int
    L.qlora_bf16_fwd.argtypes = [vp, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp]
    L.qlora_bf16_dx.restype = ctypes.c_int
    L.qlora_bf16_dx.argtypes = [vp, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp, sz, vp]
    L.qlora_nf4_dx.restype = ctypes.c_int
    L.qlora_nf4_dx.argtypes = [W, vp, i64, vp, vp, i32, f32, vp, vp]
    Wg = ctypes.POINTER(Nf4WeightDesc)
    L.qlora_group_fwd.restype = ctypes.c_int
    L.qlora_group_fwd.argtypes = [Wg, i32, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    L.qlora_group_bwd.restype = ctypes.c_int
    L.qlora_group_bwd.argtypes = [Wg, i32, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    for name in ("qlora_group_dequant", "qlora_group_dequant_t"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [Wg, i32, vp, vp]
    L.qlora_bf16_group_fwd.restype = ctypes.c_int
    L.qlora_bf16_group_fwd.argtypes = [vp, i32, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp]
    L.qlora_bf16_group_dx.restype = ctypes.c_int
    L.qlora_bf16_group_dx.argtypes = [vp, i32, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp, sz, vp]
    L.qlora_group_lora_dy_b.restype = ctypes.c_int
    L.qlora_group_lora_dy_b.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, sz, vp]
    L.qlora_group_lora_grads.restype = ctypes.c_int
    L.qlora_group_lora_grads.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, f32, vp, vp, vp, sz, vp]
    L.qlora_level_table_id.restype = ctypes.c_int
    L.qlora_level_table_id.argtypes = [i32, i32, ctypes.POINTER(ctypes.c_uint64)]
    L.qlora_qtensor_header_write.restype = ctypes.c_int
    L.qlora_qtensor_header_write.argtypes = [ctypes.POINTER(Nf4WeightDesc), ctypes.c_char_p, sz]
    L.qlora_qtensor_header_read.restype = ctypes.c_int
    L.qlora_qtensor_header_read.argtypes = [ctypes.c_char_p, sz, ctypes.POINTER(Nf4WeightDesc),
                                            ctypes.POINTER(ctypes.c_uint64)]
    _lib = L
    return L


def check(status, what):
    if status != QLORA_OK:
        raise QloraError(status, what)
