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
from . import debug as _debug
from ._lib import GemvJobDesc, GemvPlanDesc, Nf4WeightDesc, PagedLayoutDesc, PagedTensorDesc, lib
from ._lib import check as _check_status

BLOCKSIZE = 64
GROUP_BLOCKS = 256


def check(status, what):
    """Raise QloraError for a failed call; under QLORA_DEBUG=1 also
    synchronize and check the guard bands of the binding's buffers."""
    _check_status(status, what)
    if _debug.ENABLED:
        _debug.after_call(what)


def _empty(*shape, dtype, device):
    """An output or workspace buffer (guarded under QLORA_DEBUG=1); the
    shape is given as sizes or as one tuple, as for torch.empty."""
    if len(shape) == 1 and isinstance(shape[0], (tuple, list, torch.Size)):
        shape = tuple(shape[0])
    return _debug.empty(tuple(int(d) for d in shape), dtype, device)


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
# qlora_absmax_format values (second-level code of the block constants)
ABSMAX_FORMATS = {"linear": 0, "fp8": 1}


def _absfmt(name):
    if name not in ABSMAX_FORMATS:
        raise ValueError(f"unknown absmax format {name!r}: one of {sorted(ABSMAX_FORMATS)}")
    return ABSMAX_FORMATS[name]


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
    return _empty(nbytes, dtype=torch.uint8, device=device)


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
    absmax_format: str = "linear"   # "linear" or "fp8"

    def desc(self) -> Nf4WeightDesc:
        return Nf4WeightDesc(self.rows, self.cols, BLOCKSIZE, GROUP_BLOCKS, self.codes.data_ptr(),
                             self.absmax_q.data_ptr(), self.group_scale.data_ptr(), _codebook(self.codebook),
                             _absfmt(self.absmax_format))

    @staticmethod
    def empty(rows, cols, device, codebook="nf4", absmax_format="linear"):
        c, a, s = sizes(rows, cols)
        return QuantizedWeight(rows, cols,
                               _empty(c, dtype=torch.uint8, device=device),
                               _empty(a, dtype=torch.uint8, device=device),
                               _empty(s // 4, dtype=torch.float32, device=device), codebook, absmax_format)

    def nbytes(self):
        return self.codes.numel() + self.absmax_q.numel() + 4 * self.group_scale.numel()


def save_quantized(q: QuantizedWeight, path) -> None:
    """Write q to a file: the library's header (sizes, codebook, second-level
    format and the digest of their level tables), then codes, absmax_q and
    group_scale as stored.  Reading it back gives the same bytes."""
    d = q.desc()
    hdr = ctypes.create_string_buffer(_lib.QTENSOR_HEADER_BYTES)
    check(lib().qlora_qtensor_header_write(ctypes.byref(d), hdr, len(hdr)), "qlora_qtensor_header_write")
    c, a, s = sizes(q.rows, q.cols)
    arrays = ((q.codes, torch.uint8, c), (q.absmax_q, torch.uint8, a), (q.group_scale, torch.float32, s // 4))
    for t, dtype, n in arrays:
        if t.dtype != dtype or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"quantized weight arrays do not match its {q.rows} x {q.cols} sizes")
    with open(path, "wb") as f:
        f.write(hdr.raw)
        for t, _, _ in arrays:
            f.write(t.detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())


def load_quantized(path, device) -> QuantizedWeight:
    """Read a weight written by save_quantized onto `device`.  Raises
    QloraError (QLORA_E_TABLE) when the file was written with level tables
    other than this library's, QLORA_E_FORMAT when it is not such a file."""
    with open(path, "rb") as f:
        blob = f.read()
    d = Nf4WeightDesc()
    payload = ctypes.c_uint64()
    check(lib().qlora_qtensor_header_read(blob, len(blob), ctypes.byref(d), ctypes.byref(payload)),
          "qlora_qtensor_header_read")
    h = _lib.QTENSOR_HEADER_BYTES
    if len(blob) != h + payload.value:
        raise _lib.QloraError(_lib.QLORA_E_FORMAT, f"load_quantized: {path} holds {len(blob) - h} payload "
                                                   f"bytes, its header says {payload.value}")
    c, a, s = sizes(d.rows, d.cols)
    raw = torch.frombuffer(bytearray(blob[h:]), dtype=torch.uint8)
    names = {v: k for k, v in CODEBOOKS.items()}
    fmts = {v: k for k, v in ABSMAX_FORMATS.items()}
    return QuantizedWeight(int(d.rows), int(d.cols), raw[:c].clone().to(device), raw[c:c + a].clone().to(device),
                           raw[c + a:c + a + s].clone().view(torch.float32).to(device),
                           names[d.codebook], fmts[d.absmax_format])


def quantize(W: torch.Tensor, out: Optional[QuantizedWeight] = None,
             codebook: Optional[str] = None, absmax_format: Optional[str] = None) -> QuantizedWeight:
    """bf16 W [rows x cols] -> 4-bit codes + 8-bit absmax codes + fp32 group
    scales.  The codebook and the second-level format are the ones named,
    else out's, else NF4 and linear; the result records them."""
    _need(W, torch.bfloat16, "W")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    q = out if out is not None else QuantizedWeight.empty(rows, cols, W.device)
    if codebook is not None:
        _codebook(codebook)
        q.codebook = codebook
    if absmax_format is not None:
        _absfmt(absmax_format)
        q.absmax_format = absmax_format
    d = q.desc()
    check(lib().qlora_quantize(_ptr(W), ctypes.byref(d), _stream()), "qlora_quantize")
    return q


def dequant(q: QuantizedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """4-bit weight -> bf16 [rows x cols], with its codebook."""
    if out is None:
        out = _empty(q.rows, q.cols, dtype=torch.bfloat16, device=q.codes.device)
    _need(out, torch.bfloat16, "out")
    d = q.desc()
    check(lib().qlora_dequant(ctypes.byref(d), _ptr(out), _stream()), "qlora_dequant")
    return out


def dequant_t(q: QuantizedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """4-bit weight -> its transpose in bf16, [cols x rows]."""
    if out is None:
        out = _empty(q.cols, q.rows, dtype=torch.bfloat16, device=q.codes.device)
    _need(out, torch.bfloat16, "out", (q.cols, q.rows))
    d = q.desc()
    check(lib().qlora_dequant_t(ctypes.byref(d), _ptr(out), _stream()), "qlora_dequant_t")
    return out


PATHS = ("auto", "fused")


def _op(path, staged_op, fused_op):
    if path not in PATHS:
        raise ValueError(f"path must be one of {PATHS}, got {path!r}")
    return staged_op if path == "auto" else fused_op


def linear_fwd(q: QuantizedWeight, X: torch.Tensor, A=None, B=None, alpha: float = 0.0,
               save_u: bool = False, out=None, u_out=None, ws=None, path: str = "auto"):
    """Y = X deq(W)^T + (alpha/r) (X A^T) B^T.  Returns Y, or (Y, U) with save_u.

    path "auto" sizes the workspace for the staged path (the library takes it
    from 1024 tokens on: W dequantized once, then the dense bf16 product);
    "fused" sizes it for the fused path only (W decoded inside the product)."""
    _need(X, torch.bfloat16, "X")
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    if r:
        _need(A, torch.bfloat16, "A", (r, q.cols))
        _need(B, torch.bfloat16, "B", (q.rows, r))
    Y = out if out is not None else _empty(M, q.rows, dtype=torch.bfloat16, device=X.device)
    U = None
    if save_u and r:
        U = u_out if u_out is not None else _empty(M, r, dtype=torch.bfloat16, device=X.device)
    nbytes = workspace_bytes(_op(path, _lib.QLORA_OP_FWD, _lib.QLORA_OP_FWD_FUSED), M, q.rows, q.cols, r)
    if ws is None:
        ws = workspace(nbytes, X.device)
    elif ws.numel() > nbytes:
        ws = ws[:nbytes]
    d = q.desc()
    check(lib().qlora_linear_fwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y),
                                 _ptr(U), _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "qlora_linear_fwd")
    return (Y, U) if save_u else Y


def linear_fwd_noalloc(q: QuantizedWeight, X: torch.Tensor, A=None, B=None, alpha: float = 0.0,
                       save_u: bool = False, out=None, u_out=None):
    """linear_fwd through qlora_linear_fwd_noalloc: the library's scratch
    array replaces the workspace, so only the outputs (when not given) are
    allocated here.  Returns Y, or (Y, U) with save_u."""
    _need(X, torch.bfloat16, "X")
    M = X.shape[0]
    r = 0 if A is None else A.shape[0]
    if r:
        _need(A, torch.bfloat16, "A", (r, q.cols))
        _need(B, torch.bfloat16, "B", (q.rows, r))
    Y = out if out is not None else _empty(M, q.rows, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", (M, q.rows))
    U = None
    if save_u and r:
        U = u_out if u_out is not None else _empty(M, r, dtype=torch.bfloat16, device=X.device)
        _need(U, torch.bfloat16, "U", (M, r))
    d = q.desc()
    check(lib().qlora_linear_fwd_noalloc(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y),
                                         _ptr(U), _stream()), "qlora_linear_fwd_noalloc")
    return (Y, U) if save_u else Y


def linear_bwd(q: QuantizedWeight, X: torch.Tensor, dY: torch.Tensor, A=None, B=None, alpha: float = 0.0,
               U: Optional[torch.Tensor] = None, need_dx: bool = True, dX=None, dA=None, dB=None, ws=None,
               path: str = "auto"):
    """Returns (dX, dA, dB): dX bf16 [M x K] (or None), dA [r x K] and dB [N x r] fp32 (or None).
    path as in linear_fwd."""
    _need(dY, torch.bfloat16, "dY")
    M = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    if r:
        _need(X, torch.bfloat16, "X", (M, q.cols))
        _need(A, torch.bfloat16, "A", (r, q.cols))
        _need(B, torch.bfloat16, "B", (q.rows, r))
        dA = dA if dA is not None else _empty(r, q.cols, dtype=torch.float32, device=dY.device)
        dB = dB if dB is not None else _empty(q.rows, r, dtype=torch.float32, device=dY.device)
    else:
        dA = dB = None
    if need_dx:
        dX = dX if dX is not None else _empty(M, q.cols, dtype=torch.bfloat16, device=dY.device)
    else:
        dX = None
    nbytes = workspace_bytes(_op(path, _lib.QLORA_OP_BWD, _lib.QLORA_OP_BWD_FUSED), M, q.rows, q.cols, r)
    if ws is None:
        ws = workspace(nbytes, dY.device)
    elif ws.numel() > nbytes:
        ws = ws[:nbytes]
    d = q.desc()
    check(lib().qlora_linear_bwd(ctypes.byref(d), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(alpha),
                                 _ptr(U), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream()),
          "qlora_linear_bwd")
    return dX, dA, dB


def _group_descs(qs: Sequence[QuantizedWeight]):
    if not qs:
        raise ValueError("a group needs at least one weight")
    arr = (Nf4WeightDesc * len(qs))()
    for i, q in enumerate(qs):
        arr[i] = q.desc()
    return arr


def group_fwd(qs: Sequence[QuantizedWeight], X: torch.Tensor, A=None, B=None, alpha: float = 0.0,
              save_u: bool = False, out=None, u_out=None, ws=None):
    """G linears that read the same X (q/k/v, gate/up) in one call.

    A [G r x K] and B [G N x r] are the G adapters stacked; returns Y
    [M x G N] (Y_g in columns g N ..), or (Y, U) with U [M x G r]."""
    _need(X, torch.bfloat16, "X")
    G, N, K, M = len(qs), qs[0].rows, qs[0].cols, X.shape[0]
    r = 0 if A is None else A.shape[0] // G
    if A is not None:
        _need(A, torch.bfloat16, "A", (G * r, K))
        _need(B, torch.bfloat16, "B", (G * N, r))
    Y = out if out is not None else _empty(M, G * N, dtype=torch.bfloat16, device=X.device)
    U = None
    if save_u and r:
        U = u_out if u_out is not None else _empty(M, G * r, dtype=torch.bfloat16, device=X.device)
    nbytes = workspace_bytes(_lib.QLORA_OP_GROUP_FWD, M, N, K, r, G)
    if ws is None:
        ws = workspace(nbytes, X.device)
    elif ws.numel() > nbytes:
        ws = ws[:nbytes]
    descs = _group_descs(qs)
    check(lib().qlora_group_fwd(descs, G, _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(U),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "qlora_group_fwd")
    return (Y, U) if save_u else Y


def group_bwd(qs: Sequence[QuantizedWeight], X: torch.Tensor, dY: torch.Tensor, A=None, B=None,
              alpha: float = 0.0, U: Optional[torch.Tensor] = None, need_dx: bool = True, dX=None, dA=None,
              dB=None, ws=None):
    """Backward of group_fwd: dY [M x G N]; returns (dX [M x K] bf16 or None,
    dA [G r x K] fp32, dB [G N x r] fp32) (the last two None without adapters)."""
    _need(dY, torch.bfloat16, "dY")
    G, N, K, M = len(qs), qs[0].rows, qs[0].cols, dY.shape[0]
    _need(dY, torch.bfloat16, "dY", (M, G * N))
    r = 0 if A is None else A.shape[0] // G
    if r:
        _need(X, torch.bfloat16, "X", (M, K))
        _need(A, torch.bfloat16, "A", (G * r, K))
        _need(B, torch.bfloat16, "B", (G * N, r))
        dA = dA if dA is not None else _empty(G * r, K, dtype=torch.float32, device=dY.device)
        dB = dB if dB is not None else _empty(G * N, r, dtype=torch.float32, device=dY.device)
    else:
        dA = dB = None
    if need_dx:
        dX = dX if dX is not None else _empty(M, K, dtype=torch.bfloat16, device=dY.device)
    else:
        dX = None
    nbytes = workspace_bytes(_lib.QLORA_OP_GROUP_BWD, M, N, K, r, G)
    if ws is None:
        ws = workspace(nbytes, dY.device)
    elif ws.numel() > nbytes:
        ws = ws[:nbytes]
    descs = _group_descs(qs)
    check(lib().qlora_group_bwd(descs, G, _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(U),
                                _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream()),
          "qlora_group_bwd")
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
    y = j.y if j.y is not None else _empty(shape, dtype=torch.bfloat16, device=j.x.device)
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
    U = U if U is not None else _empty(M, r, dtype=torch.bfloat16, device=X.device)
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
    G = G if G is not None else _empty(M, r, dtype=torch.bfloat16, device=dY.device)
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
    dA = dA if dA is not None else _empty(r, K, dtype=torch.float32, device=X.device)
    dB = dB if dB is not None else _empty(N, r, dtype=torch.float32, device=X.device)
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
    Y = out if out is not None else _empty(M, q.rows, dtype=torch.bfloat16, device=X.device)
    d = q.desc()
    check(lib().qlora_nf4_fwd(ctypes.byref(d), _ptr(X), M, _ptr(U), _ptr(B), r, float(alpha), _ptr(Y),
                              _stream()), "qlora_nf4_fwd")
    return Y


def bf16_fwd(Wd: torch.Tensor, X, U=None, B=None, alpha: float = 0.0, out=None):
    """The dense forward GEMM on a dequantized weight Wd [N x K] (bf16):
    Y = X Wd^T + s U B^T."""
    _need(Wd, torch.bfloat16, "Wd")
    _need(X, torch.bfloat16, "X")
    N, K = Wd.shape
    M = X.shape[0]
    r = 0 if U is None else U.shape[1]
    if r:
        _need(U, torch.bfloat16, "U", (M, r))
        _need(B, torch.bfloat16, "B", (N, r))
    Y = out if out is not None else _empty(M, N, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", (M, N))
    check(lib().qlora_bf16_fwd(_ptr(Wd), N, K, _ptr(X), M, _ptr(U), _ptr(B), r, float(alpha), _ptr(Y), _stream()),
          "qlora_bf16_fwd")
    return Y


def bf16_dx(WdT: torch.Tensor, dY, G=None, A=None, alpha: float = 0.0, out=None, ws=None):
    """The dense backward GEMM on the transposed bf16 weight WdT [K x N]:
    dX = dY WdT^T + s G A.  Shapes with few output tiles and a long
    contraction split it in ws (allocated here when not given)."""
    _need(WdT, torch.bfloat16, "WdT")
    _need(dY, torch.bfloat16, "dY")
    K, N = WdT.shape
    M = dY.shape[0]
    r = 0 if G is None else G.shape[1]
    if r:
        _need(G, torch.bfloat16, "G", (M, r))
        _need(A, torch.bfloat16, "A", (r, K))
    dX = out if out is not None else _empty(M, K, dtype=torch.bfloat16, device=dY.device)
    _need(dX, torch.bfloat16, "dX", (M, K))
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_BF16_DX, M, N, K, r, 1), dY.device)
    check(lib().qlora_bf16_dx(_ptr(WdT), N, K, _ptr(dY), M, _ptr(G), _ptr(A), r, float(alpha), _ptr(dX),
                              _ptr(ws), 0 if ws is None else ws.numel(), _stream()), "qlora_bf16_dx")
    return dX


def group_dequant(qs: Sequence[QuantizedWeight], out=None, transposed=False):
    """The G weights dequantized into one stack [G N x K], or side by side
    transposed [K x G N]."""
    G, N, K = len(qs), qs[0].rows, qs[0].cols
    shape = (K, G * N) if transposed else (G * N, K)
    out = out if out is not None else _empty(*shape, dtype=torch.bfloat16, device=qs[0].codes.device)
    _need(out, torch.bfloat16, "out", shape)
    fn = lib().qlora_group_dequant_t if transposed else lib().qlora_group_dequant
    check(fn(_group_descs(qs), G, _ptr(out), _stream()),
          "qlora_group_dequant_t" if transposed else "qlora_group_dequant")
    return out


def bf16_group_fwd(Wd: torch.Tensor, G: int, X, U=None, B=None, alpha: float = 0.0, out=None):
    """The group's dense forward product on the stack Wd [G N x K]:
    Y [M x G N] = X Wd^T + s (U_g B_g^T side by side)."""
    _need(Wd, torch.bfloat16, "Wd")
    _need(X, torch.bfloat16, "X")
    N, K, M = Wd.shape[0] // G, Wd.shape[1], X.shape[0]
    r = 0 if U is None else U.shape[1] // G
    if r:
        _need(U, torch.bfloat16, "U", (M, G * r))
        _need(B, torch.bfloat16, "B", (G * N, r))
    Y = out if out is not None else _empty(M, G * N, dtype=torch.bfloat16, device=X.device)
    _need(Y, torch.bfloat16, "Y", (M, G * N))
    check(lib().qlora_bf16_group_fwd(_ptr(Wd), G, N, K, _ptr(X), M, _ptr(U), _ptr(B), r, float(alpha), _ptr(Y),
                                     _stream()), "qlora_bf16_group_fwd")
    return Y


def bf16_group_dx(WdT: torch.Tensor, G: int, dY, Gm=None, A=None, alpha: float = 0.0, out=None, ws=None):
    """The group's dense dX product on WdT [K x G N]: dX = dY WdT^T + s Gm A
    (ws as for bf16_dx)."""
    _need(WdT, torch.bfloat16, "WdT")
    _need(dY, torch.bfloat16, "dY")
    K, N, M = WdT.shape[0], WdT.shape[1] // G, dY.shape[0]
    r = 0 if Gm is None else Gm.shape[1] // G
    if r:
        _need(Gm, torch.bfloat16, "Gm", (M, G * r))
        _need(A, torch.bfloat16, "A", (G * r, K))
    dX = out if out is not None else _empty(M, K, dtype=torch.bfloat16, device=dY.device)
    _need(dX, torch.bfloat16, "dX", (M, K))
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_BF16_DX, M, N, K, r, G), dY.device)
    check(lib().qlora_bf16_group_dx(_ptr(WdT), G, N, K, _ptr(dY), M, _ptr(Gm), _ptr(A), r, float(alpha), _ptr(dX),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream()), "qlora_bf16_group_dx")
    return dX


def group_lora_dy_b(dY, B, G: int, Gm=None, ws=None):
    """Gm [M x G r]: columns g r .. are dY_g B_g (bf16)."""
    _need(dY, torch.bfloat16, "dY")
    M, N = dY.shape[0], dY.shape[1] // G
    r = B.shape[1]
    _need(B, torch.bfloat16, "B", (G * N, r))
    Gm = Gm if Gm is not None else _empty(M, G * r, dtype=torch.bfloat16, device=dY.device)
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_GROUP_LORA, M, N, 64, r, G), dY.device)
    check(lib().qlora_group_lora_dy_b(_ptr(dY), _ptr(B), M, N, r, G, _ptr(Gm), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream()), "qlora_group_lora_dy_b")
    return Gm


def group_lora_grads(X, dY, U, Gm, G: int, alpha, dA=None, dB=None, ws=None):
    """dA [G r x K] = s Gm^T X and dB [G N x r], dB_g = s dY_g^T U_g (fp32)."""
    M, K = X.shape
    N, r = dY.shape[1] // G, U.shape[1] // G
    for t, n, shp in ((X, "X", (M, K)), (dY, "dY", (M, G * N)), (U, "U", (M, G * r)), (Gm, "Gm", (M, G * r))):
        _need(t, torch.bfloat16, n, shp)
    dA = dA if dA is not None else _empty(G * r, K, dtype=torch.float32, device=X.device)
    dB = dB if dB is not None else _empty(G * N, r, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(workspace_bytes(_lib.QLORA_OP_GROUP_LORA, M, N, K, r, G), X.device)
    check(lib().qlora_group_lora_grads(_ptr(X), _ptr(dY), _ptr(U), _ptr(Gm), M, N, K, r, G, float(alpha), _ptr(dA),
                                       _ptr(dB), _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "qlora_group_lora_grads")
    return dA, dB


def nf4_dx(q: QuantizedWeight, dY, G=None, A=None, alpha: float = 0.0, out=None):
    """The fused backward GEMM: dX = dY deq(W) + s G A."""
    _need(dY, torch.bfloat16, "dY")
    M = dY.shape[0]
    r = 0 if G is None else G.shape[1]
    dX = out if out is not None else _empty(M, q.cols, dtype=torch.bfloat16, device=dY.device)
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


class PagedAdamW:
    """AdamW with the moments in a pinned host backing store, paged through a
    device buffer of `budget_bytes` (qlora_paged_adamw).  params / grads:
    lists of fp32 device tensors (grads refilled by the caller before each
    step); p_bf16: optional matching bf16 device tensors.  The host moments
    are allocated pinned here, zero; step() runs one update on the current
    stream, with the host <-> device copies on copy_stream (a torch Stream)."""

    def __init__(self, params, grads, budget_bytes, p_bf16=None, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8,
                 weight_decay=0.0, copy_stream=None):
        n = len(params)
        self.params, self.grads = list(params), list(grads)
        self.p_bf16 = list(p_bf16) if p_bf16 is not None else [None] * n
        for i in range(n):
            p, g = self.params[i], self.grads[i]
            if p.dtype != torch.float32 or g.dtype != torch.float32 or not p.is_cuda or not g.is_cuda:
                raise ValueError("params and grads must be float32 GPU tensors")
            if not p.is_contiguous() or not g.is_contiguous() or p.numel() != g.numel():
                raise ValueError("params and grads must be contiguous and of equal size")
            if self.p_bf16[i] is not None:
                _need(self.p_bf16[i], torch.bfloat16, "p_bf16")
        self.m = [torch.zeros(p.numel(), dtype=torch.float32, pin_memory=True) for p in self.params]
        self.v = [torch.zeros(p.numel(), dtype=torch.float32, pin_memory=True) for p in self.params]
        self.descs = (PagedTensorDesc * n)()
        for i in range(n):
            pb = self.p_bf16[i]
            self.descs[i] = PagedTensorDesc(self.params[i].data_ptr(), None if pb is None else pb.data_ptr(),
                                            self.grads[i].data_ptr(), self.m[i].data_ptr(), self.v[i].data_ptr(),
                                            self.params[i].numel())
        self.n = n
        lay = PagedLayoutDesc()
        check(lib().qlora_paged_layout_of(self.descs, n, int(budget_bytes), ctypes.byref(lay)), "qlora_paged_layout_of")
        self.layout = dict(resident=lay.resident, resident_bytes=lay.resident_bytes, chunk=lay.chunk,
                           staging_bytes=lay.staging_bytes)
        self.budget = int(budget_bytes)
        self.ws = _empty(max(self.budget, 256), dtype=torch.uint8, device=self.params[0].device)
        self.hp = (lr, beta1, beta2, eps, weight_decay)
        self.copy_stream = copy_stream
        self.t = 0

    def step(self, store=False):
        """One update; store=True also writes the resident moments back to the host."""
        self.t += 1
        flags = (_lib.QLORA_PAGED_LOAD if self.t == 1 else 0) | (_lib.QLORA_PAGED_STORE if store else 0)
        cs = None if self.copy_stream is None else ctypes.c_void_p(self.copy_stream.cuda_stream)
        check(lib().qlora_paged_adamw(self.descs, self.n, ctypes.c_void_p(self.ws.data_ptr()), self.budget,
                                      *[float(x) for x in self.hp], self.t, flags, _stream(), cs),
              "qlora_paged_adamw")
