"""Python binding of libqlora: argument marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  All tensors must be on the
GPU; there is no CPU path.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import GemvJobDesc, GemvPlanDesc, Nf4WeightDesc, check, lib

BLOCKSIZE = 64
GROUP_BLOCKS = 256


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def sizes(rows, cols):
    """(codes bytes, absmax_q bytes, group_scale bytes) of a rows x cols weight."""
    c, a, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().qlora_sizes(rows, cols, BLOCKSIZE, GROUP_BLOCKS, ctypes.byref(c), ctypes.byref(a),
                            ctypes.byref(s)), "qlora_sizes")
    return c.value, a.value, s.value


def nf4_levels():
    buf = (ctypes.c_float * 16)()
    lib().qlora_nf4_levels(buf)
    return torch.tensor(list(buf), dtype=torch.float32)


# qlora_codebook values
CODEBOOKS = {"nf4": 0, "fp4": 1, "int4": 2}


def _codebook(name):
    if name not in CODEBOOKS:
        raise ValueError(f"unknown codebook {name!r}: one of {sorted(CODEBOOKS)}")
    return CODEBOOKS[name]


def codebook_levels(name="nf4"):
    """The 16 fp32 levels of a codebook ("nf4", "fp4", "int4") as the library holds them."""
    buf = (ctypes.c_float * 16)()
    check(lib().qlora_codebook_levels(_codebook(name), buf), "qlora_codebook_levels")
    return torch.tensor(list(buf), dtype=torch.float32)


def workspace_bytes(op, M=0, N=0, K=0, r=0, njobs=0):
    return int(lib().qlora_workspace_bytes(op, M, N, K, r, njobs))


def workspace(nbytes, device):
    """A workspace tensor (uint8) of at least nbytes, or None when 0."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@dataclass
class QuantizedWeight:
    """A 4-bit (NF4 unless another codebook is named) + double-quantized
    weight [rows x cols] held in torch tensors."""
    rows: int
    cols: int
    codes: torch.Tensor        # uint8 [ceil(rows*cols/2)]
    absmax_q: torch.Tensor     # uint8 [nb]
    group_scale: torch.Tensor  # float32 [ng]
    codebook: str = "nf4"      # "nf4", "fp4" or "int4"

    def desc(self) -> Nf4WeightDesc:
        return Nf4WeightDesc(self.rows, self.cols, BLOCKSIZE, GROUP_BLOCKS, self.codes.data_ptr(),
                             self.absmax_q.data_ptr(), self.group_scale.data_ptr(), _codebook(self.codebook))

    @staticmethod
    def empty(rows, cols, device, codebook="nf4"):
        c, a, s = sizes(rows, cols)
        return QuantizedWeight(rows, cols,
                               torch.empty(c, dtype=torch.uint8, device=device),
                               torch.empty(a, dtype=torch.uint8, device=device),
                               torch.empty(s // 4, dtype=torch.float32, device=device), codebook)

    def nbytes(self):
        return self.codes.numel() + self.absmax_q.numel() + 4 * self.group_scale.numel()


def quantize(W: torch.Tensor, out: Optional[QuantizedWeight] = None,
             codebook: Optional[str] = None) -> QuantizedWeight:
    """bf16 W [rows x cols] -> 4-bit codes + 8-bit absmax codes + fp32 group
    scales.  The codebook is the one named, else out's, else NF4; the
    result records it."""
    _need(W, torch.bfloat16, "W")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    q = out if out is not None else QuantizedWeight.empty(rows, cols, W.device)
    if codebook is not None:
        _codebook(codebook)
        q.codebook = codebook
    d = q.desc()
    check(lib().qlora_quantize(_ptr(W), ctypes.byref(d), _stream()), "qlora_quantize")
    return q


def dequant(q: QuantizedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """4-bit weight -> bf16 [rows x cols], with its codebook."""
    if out is None:
        out = torch.empty(q.rows, q.cols, dtype=torch.bfloat16, device=q.codes.device)
    _need(out, torch.bfloat16, "out")
    d = q.desc()
    check(lib().qlora_dequant(ctypes.byref(d), _ptr(out), _stream()), "qlora_dequant")
    return out


def linear_fwd(q: QuantizedWeight, X: torch.Tensor, A=None, B=None, alpha: float = 0.0,
               save_u: bool = False, out=None, u_out=None, ws=None):
    """Y = X deq(W)^T + (alpha/r) (X A^T) B^T.  Returns Y, or (Y, U) with save_u."""
    _need(X, torch.bfloat16, "X")
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    if r:
        _need(A, torch.bfloat16, "A", (r, q.cols))
        _need(B, torch.bfloat16, "B", (q.rows, r))
    Y = out if out is not None else torch.empty(M, q.rows, dtype=torch.bfloat16, device=X.device)
    U = None
    if save_u and r:
        U = u_out if u_out is not None else torch.empty(M, r, dtype=torch.bfloat16, device=X.device)
    nbytes = workspace_bytes(_lib.QLORA_OP_FWD, M, q.rows, q.cols, r)
    if ws is None:
        ws = workspace(nbytes, X.device)
    d = q.desc()
    check(lib().qlora_linear_fwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y),
                                 _ptr(U), _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "qlora_linear_fwd")
    return (Y, U) if save_u else Y


def linear_bwd(q: QuantizedWeight, X: torch.Tensor, dY: torch.Tensor, A=None, B=None, alpha: float = 0.0,
               U: Optional[torch.Tensor] = None, need_dx: bool = True, dX=None, dA=None, dB=None, ws=None):
    """Returns (dX, dA, dB): dX bf16 [M x K] (or None), dA [r x K] and dB [N x r] fp32 (or None)."""
    _need(dY, torch.bfloat16, "dY")
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    if r:
        _need(X, torch.bfloat16, "X", (M, q.cols))
        _need(A, torch.bfloat16, "A", (r, q.cols))
        _need(B, torch.bfloat16, "B", (q.rows, r))
        dA = dA if dA is not None else torch.empty(r, q.cols, dtype=torch.float32, device=dY.device)
        dB = dB if dB is not None else torch.empty(q.rows, r, dtype=torch.float32, device=dY.device)
    else:
        dA = dB = None
    if need_dx:
        dX = dX if dX is not None else torch.empty(M, q.cols, dtype=torch.bfloat16, device=dY.device)
    else:
        dX = None
    nbytes = workspace_bytes(_lib.QLORA_OP_BWD, M, q.rows, q.cols, r)
    if ws is None:
        ws = workspace(nbytes, dY.device)
    d = q.desc()
    check(lib().qlora_linear_bwd(ctypes.byref(d), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(alpha),
                                 _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream()),
          "qlora_linear_bwd")
    return dX, dA, dB


@dataclass
class GemvJob:
    """One decode product: x is [cols] (one token) or [m x cols] (m <= 16
    tokens); y, when given, has the matching shape [rows] or [m x rows]."""
    q: QuantizedWeight
    x: torch.Tensor
    A: Optional[torch.Tensor] = None
    B: Optional[torch.Tensor] = None
    alpha: float = 0.0
    y: Optional[torch.Tensor] = None


class GemvPlan:
    """A prepared decode call: the job table is written into the workspace once
    (qlora_gemv_prepare, on the current stream); calling the plan enqueues
    qlora_gemv_run.  The tensors the jobs name must stay alive and in place."""

    def __init__(self, jobs: Sequence[GemvJob], ws=None):
        n = len(jobs)
        self._descs = (Nf4WeightDesc * n)()
        self._arr = (GemvJobDesc * n)()
        self.outputs = []
        self._keep = list(jobs)
        for i, j in enumerate(jobs):
            self._descs[i] = j.q.desc()
            self._arr[i], y = _gemv_desc(j, self._descs[i])
            self.outputs.append(y)
        self.n = n
        nbytes = workspace_bytes(_lib.QLORA_OP_GEMV, M=max(_tokens(j) for j in jobs), N=max(j.q.rows for j in jobs),
                                 K=max(j.q.cols for j in jobs), njobs=n)
        self.ws = ws if ws is not None else workspace(nbytes, jobs[0].x.device)
        self._plan = GemvPlanDesc()
        check(lib().qlora_gemv_prepare(self._arr, n, _ptr(self.ws), 0 if self.ws is None else self.ws.numel(),
                                       ctypes.byref(self._plan), _stream()), "qlora_gemv_prepare")

    def __call__(self):
        check(lib().qlora_gemv_run(ctypes.byref(self._plan), _stream()), "qlora_gemv_run")
        return self.outputs


def _tokens(j):
    return 1 if j.x.dim() == 1 else int(j.x.shape[0])


def _gemv_desc(j, desc):
    """(job descriptor, y) for one GemvJob; desc must outlive the call."""
    m = _tokens(j)
    one = j.x.dim() == 1
    _need(j.x, torch.bfloat16, "x", (j.q.cols,) if one else (m, j.q.cols))
    r = 0 if j.A is None else j.A.shape[0]
    if r:
        _need(j.A, torch.bfloat16, "A", (r, j.q.cols))
        _need(j.B, torch.bfloat16, "B", (j.q.rows, r))
    shape = (j.q.rows,) if one else (m, j.q.rows)
    y = j.y if j.y is not None else torch.empty(shape, dtype=torch.bfloat16, device=j.x.device)
    _need(y, torch.bfloat16, "y", shape)
    return GemvJobDesc(ctypes.pointer(desc), j.x.data_ptr(), None if r == 0 else j.A.data_ptr(),
                       None if r == 0 else j.B.data_ptr(), r, float(j.alpha), y.data_ptr(), m), y


def gemv(jobs: Sequence[GemvJob], ws=None):
    """Decode (one token or a batch of up to 16 per job) for independent
    linears; returns the list of y tensors."""
    n = len(jobs)
    descs = (Nf4WeightDesc * n)()
    arr = (GemvJobDesc * n)()
    outs = []
    for i, j in enumerate(jobs):
        descs[i] = j.q.desc()
        arr[i], y = _gemv_desc(j, descs[i])
        outs.append(y)
    nbytes = workspace_bytes(_lib.QLORA_OP_GEMV, M=max(_tokens(j) for j in jobs), N=max(j.q.rows for j in jobs),
                             K=max(j.q.cols for j in jobs), njobs=n)
    if ws is None:
        ws = workspace(nbytes, jobs[0].x.device)
    check(lib().qlora_gemv(arr, n, _ptr(ws), 0 if ws is None else ws.numel(), _stream()), "qlora_gemv")
    return outs


# ---- building blocks (the two fused GEMMs and the LoRA side products) ----

def lora_down(X, A, U=None, ws=None):
    """U [M x r] = X A^T (bf16)."""
    _need(X, torch.bfloat16, "X")
    M, K = X.shape
    r = A.shape[0]
    _need(A, torch.bfloat16, "A", (r, K))
    U = U if U is not None else torch.empty(M, r, dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_LORA, M, 8, K, r), X.device)
    check(lib().qlora_lora_down(_ptr(X), _ptr(A), M, K, r, _ptr(U), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream()), "qlora_lora_down")
    return U


def lora_dy_b(dY, B, G=None, ws=None):
    """G [M x r] = dY B (bf16)."""
    _need(dY, torch.bfloat16, "dY")
    M, N = dY.shape
    r = B.shape[1]
    _need(B, torch.bfloat16, "B", (N, r))
    G = G if G is not None else torch.empty(M, r, dtype=torch.bfloat16, device=dY.device)
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_LORA, M, N, 8, r), dY.device)
    check(lib().qlora_lora_dy_b(_ptr(dY), _ptr(B), M, N, r, _ptr(G), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream()), "qlora_lora_dy_b")
    return G


def lora_grads(X, dY, U, G, alpha, dA=None, dB=None, ws=None):
    """dA [r x K] = s G^T X, dB [N x r] = s dY^T U (fp32)."""
    M, K = X.shape
    N = dY.shape[1]
    r = U.shape[1]
    for t, n, shp in ((X, "X", (M, K)), (dY, "dY", (M, N)), (U, "U", (M, r)), (G, "G", (M, r))):
        _need(t, torch.bfloat16, n, shp)
    dA = dA if dA is not None else torch.empty(r, K, dtype=torch.float32, device=X.device)
    dB = dB if dB is not None else torch.empty(N, r, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_LORA, M, N, K, r), X.device)
    check(lib().qlora_lora_grads(_ptr(X), _ptr(dY), _ptr(U), _ptr(G), M, N, K, r, float(alpha), _ptr(dA),
                                 _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "qlora_lora_grads")
    return dA, dB


def nf4_fwd(q: QuantizedWeight, X, U=None, B=None, alpha: float = 0.0, out=None):
    """The fused forward GEMM: Y = X deq(W)^T + s U B^T."""
    _need(X, torch.bfloat16, "X")
    M = X.shape[0]
    r = 0 if U is None else U.shape[1]
    Y = out if out is not None else torch.empty(M, q.rows, dtype=torch.bfloat16, device=X.device)
    d = q.desc()
    check(lib().qlora_nf4_fwd(ctypes.byref(d), _ptr(X), M, _ptr(U), _ptr(B), r, float(alpha), _ptr(Y),
                              _stream()), "qlora_nf4_fwd")
    return Y


def nf4_dx(q: QuantizedWeight, dY, G=None, A=None, alpha: float = 0.0, out=None):
    """The fused backward GEMM: dX = dY deq(W) + s G A."""
    _need(dY, torch.bfloat16, "dY")
    M = dY.shape[0]
    r = 0 if G is None else G.shape[1]
    dX = out if out is not None else torch.empty(M, q.cols, dtype=torch.bfloat16, device=dY.device)
    d = q.desc()
    check(lib().qlora_nf4_dx(ctypes.byref(d), _ptr(dY), M, _ptr(G), _ptr(A), r, float(alpha), _ptr(dX),
                             _stream()), "qlora_nf4_dx")
    return dX


def adamw(p: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, step: int, lr: float = 1e-4,
          beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
          p_bf16: Optional[torch.Tensor] = None):
    """One AdamW step in place: fp32 p, grad, m, v of one shape (device or
    pinned host memory); p_bf16 (optional, bf16) receives the bf16 copy."""
    n = p.numel()
    for t, name in ((p, "p"), (grad, "grad"), (m, "m"), (v, "v")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous float32 tensor of {n} elements")
    if p_bf16 is not None and (p_bf16.dtype != torch.bfloat16 or not p_bf16.is_contiguous() or p_bf16.numel() != n):
        raise ValueError(f"p_bf16 must be a contiguous bfloat16 tensor of {n} elements")
    check(lib().qlora_adamw(p.data_ptr(), None if p_bf16 is None else p_bf16.data_ptr(), grad.data_ptr(),
                            m.data_ptr(), v.data_ptr(), n, lr, beta1, beta2, eps, weight_decay, step, _stream()),
          "qlora_adamw")
