"""The LoRA-adapted frozen linear layer, forward and backward, in fp64.

Pages: the LoRA update is a low-rank product added to the frozen weight
(deepfa.ir "LoRA: Prerequisite"); the frozen weight is used in BFloat16 after
dequantization, the adapters are trained in 16-bit, and weight gradients are
computed only for the LoRA matrices (glossary "Definition"; deepfa.ir
"QLoRA's Working Process", steps 4-5); gradients flow through the frozen
4-bit model into the adapters (insights4ai page).

Reading R11 (orientation and scale, from the task's problem statement; the
pages name A d x r and B r x k without a scale): with W [N x K] (out x in),
X [M x K], A [r x K], B [N x r] and s = RN32(alpha / r),

    Y  = X Wd^T + s (X A^T) B^T
    dX = dY Wd + s (dY B) A
    dA = s (dY B)^T X
    dB = s dY^T (X A^T)

where Wd is the dequantized bf16 weight.  No bias, no dropout, no weight
gradient for W.  Everything is fp64 on bf16-exact inputs, with no
intermediate rounding; numpy's float64 matmul is the only library routine.
"""

import numpy as np


def lora_scale(alpha, r):
    """s = RN32(alpha / r) as a Python float (0 when r == 0)."""
    if r == 0:
        return 0.0
    return float(np.float32(np.float64(alpha) / np.float64(r)))


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def linear_fwd(Wd, X, A=None, B=None, alpha=0.0):
    """Y [M x N] = X Wd^T + s (X A^T) B^T."""
    Wd, X, A, B = _f64(Wd), _f64(X), _f64(A), _f64(B)
    Y = X @ Wd.T
    if A is not None and A.shape[0] > 0:
        s = lora_scale(alpha, A.shape[0])
        Y = Y + s * ((X @ A.T) @ B.T)
    return Y


def adapter_grads(X, dY, A, B, alpha):
    """(dA [r x K], dB [N x r]): the adapters' gradients, which do not involve
    the frozen weight."""
    X, dY, A, B = _f64(X), _f64(dY), _f64(A), _f64(B)
    s = lora_scale(alpha, A.shape[0])
    G = dY @ B                       # [M x r]
    dA = s * (G.T @ X)
    dB = s * (dY.T @ (X @ A.T))
    return dA, dB


def linear_bwd(Wd, X, dY, A=None, B=None, alpha=0.0):
    """Return (dX [M x K], dA [r x K] or None, dB [N x r] or None)."""
    Wd, X, dY, A, B = _f64(Wd), _f64(X), _f64(dY), _f64(A), _f64(B)
    dX = dY @ Wd
    if A is None or A.shape[0] == 0:
        return dX, None, None
    s = lora_scale(alpha, A.shape[0])
    dX = dX + s * ((dY @ B) @ A)
    dA, dB = adapter_grads(X, dY, A, B, alpha)
    return dX, dA, dB


def gemv(Wd, x, A=None, B=None, alpha=0.0):
    """Batch-1 decode: y [N] = Wd x + s B (A x)."""
    Wd, x, A, B = _f64(Wd), _f64(x).ravel(), _f64(A), _f64(B)
    y = Wd @ x
    if A is not None and A.shape[0] > 0:
        s = lora_scale(alpha, A.shape[0])
        y = y + s * (B @ (A @ x))
    return y
