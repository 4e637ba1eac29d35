"""Shared helpers for the parity tests (conversion, tolerances, sampling)."""

import numpy as np
import torch

import oracle

# Tolerances of the forward / backward / GEMV outputs (relative Frobenius
# error and largest element error relative to the largest reference value).
REL_FROB = 5e-3
MAX_ABS_REL = 1e-2


def bits_to_torch(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> bf16 torch tensor on device."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(device)


def torch_to_bits(t):
    """bf16 torch tensor -> uint16 numpy bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def torch_to_f64(t):
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(torch_to_bits(t)).reshape(tuple(t.shape))
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(got, ref, name=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    den = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    rel = err / den if den > 0 else err
    mx = np.max(np.abs(got - ref)) if got.size else 0.0
    ref_max = np.max(np.abs(ref)) if ref.size else 0.0
    assert rel <= REL_FROB, f"{name}: relative Frobenius error {rel:.3e} > {REL_FROB}"
    assert mx <= MAX_ABS_REL * ref_max + (0.0 if ref_max > 0 else 1e-30), \
        f"{name}: max abs error {mx:.3e} > {MAX_ABS_REL} * {ref_max:.3e}"
    return rel, mx


def oracle_quantize_rows(w_bits_flat, K, rows):
    """Oracle NF4 codes/absmax/scales + dequantized rows for selected rows.

    Groups are independent, so quantizing the group-aligned slice that covers
    a row gives the same codes as quantizing the whole tensor.
    """
    G = 64 * 256
    out = {}
    for n in rows:
        lo = (n * K) // G * G
        hi = min(w_bits_flat.size, -(-((n + 1) * K) // G) * G)
        codes, aq, s2 = oracle.quantize(w_bits_flat[lo:hi])
        deq = oracle.dequant(codes, aq, s2, hi - lo)
        out[n] = oracle.bf16_bits_to_f64(deq[n * K - lo:(n + 1) * K - lo])
    return out
