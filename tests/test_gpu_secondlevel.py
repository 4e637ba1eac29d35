"""GPU parity of the FP8 (E4M3) second level of the block constants (reading
R19, qlora_absmax_format QLORA_ABSMAX_FP8) against the fp64 oracle.

Bit-exact: NF4 codes, absmax codes, group scales and the dequantized bf16
weight (plain and transposed), on random weights, weights with outliers and
groups whose constants span four decades (where FP8 keeps what the linear
code rounds to zero).  Within the usual tolerances: the forward and backward
on both paths (fused, and staged through the dense kernel) and the decode
GEMV at one and several tokens.  One call may not mix formats.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _weights(kind, N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02
    if kind == "outliers":
        w[rng.random((N, K)) < 0.001] *= 8.0
    elif kind == "wide":   # one block per group about 1e4 times the others
        w = rng.standard_normal((N, K)) * 1e-4
        flat = w.reshape(-1)
        for g in range(0, flat.size, 64 * 256):
            flat[g:g + 64] = rng.standard_normal(min(64, flat.size - g))
    return synth.to_bf16_bits(w.astype(np.float32))


@pytest.mark.parametrize("kind", ["normal", "outliers", "wide"])
@pytest.mark.parametrize("N,K", [(256, 1024), (1000, 576), (37, 22016)])
def test_fp8_storage_and_dequant_bit_exact(kind, N, K):
    print(f"[fp8 second level] {kind} N{N} K{K}", flush=True)
    wb = _weights(kind, N, K, N + K)
    q = ops.quantize(bits_to_torch(wb), absmax_format="fp8")
    Wd = ops.dequant(q)
    Wt = ops.dequant_t(q) if N % 8 == 0 else None
    torch.cuda.synchronize()
    c, a, s = oracle.quantize(wb, absmax_format="fp8")
    assert np.array_equal(q.codes.cpu().numpy(), c)
    assert np.array_equal(q.absmax_q.cpu().numpy(), a)
    assert np.array_equal(q.group_scale.cpu().numpy().view(np.uint32), s.view(np.uint32))
    ref = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, wb.size, absmax_format="fp8")).reshape(N, K)
    assert np.array_equal(torch_to_f64(Wd), ref)
    if Wt is not None:
        assert np.array_equal(torch_to_f64(Wt), ref.T)
    if kind == "wide":   # the small constants survive (the linear code stores them as 0)
        assert np.count_nonzero(a) > 0.9 * a.size


def _case(M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    return dict(W=_weights("outliers", N, K, seed), X=g((M, K), 1.0), dY=g((M, N), 1.0), A=g((r, K), 0.2),
                B=g((N, r), 0.2), alpha=16.0)


@pytest.mark.parametrize("M,N,K,r", [(300, 1032, 1088, 64), (1100, 1088, 576, 16)])
@pytest.mark.parametrize("path", ["auto", "fused"])
def test_fp8_linear_forward_backward(M, N, K, r, path):
    print(f"[fp8 linear] M{M} N{N} K{K} r{r} {path}", flush=True)
    d = _case(M, N, K, r, seed=M + N + K)
    q = ops.quantize(bits_to_torch(d["W"]), absmax_format="fp8")
    X, A, B, dY = (bits_to_torch(d[k]) for k in ("X", "A", "B", "dY"))
    Y, U = ops.linear_fwd(q, X, A, B, d["alpha"], save_u=True, path=path)
    dX, dA, dB = ops.linear_bwd(q, X, dY, A, B, d["alpha"], U=U, path=path)
    torch.cuda.synchronize()
    c, a, s = oracle.quantize(d["W"], absmax_format="fp8")
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size, absmax_format="fp8")).reshape(N, K)
    f = lambda k: oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    Yr = oracle.linear_fwd(Wd, f("X"), f("A"), f("B"), d["alpha"])
    dXr, dAr, dBr = oracle.linear_bwd(Wd, f("X"), f("dY"), f("A"), f("B"), d["alpha"])
    for name, got, ref in (("Y", Y, Yr), ("dX", dX, dXr), ("dA", dA, dAr), ("dB", dB, dBr)):
        assert_close(torch_to_f64(got), ref, f"{name} {path}")


@pytest.mark.parametrize("m", [1, 5])
def test_fp8_decode(m):
    rng = np.random.default_rng(90 + m)
    jobs, refs = [], []
    for i, (N, K, r) in enumerate([(512, 1024, 64), (37, 22016, 16), (300, 1536, 0)]):
        wb = _weights("wide" if i == 0 else "outliers", N, K, 100 * m + i)
        x = synth.to_bf16_bits(rng.standard_normal((m, K) if m > 1 else (K,)))
        A = synth.to_bf16_bits(rng.standard_normal((r, K)) * 0.2) if r else None
        B = synth.to_bf16_bits(rng.standard_normal((N, r)) * 0.2) if r else None
        q = ops.quantize(bits_to_torch(wb), absmax_format="fp8")
        jobs.append(ops.GemvJob(q, bits_to_torch(x), bits_to_torch(A) if r else None,
                                bits_to_torch(B) if r else None, 16.0))
        c, a, s = oracle.quantize(wb, absmax_format="fp8")
        Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, wb.size, absmax_format="fp8")).reshape(N, K)
        f = lambda v: None if v is None else oracle.bf16_bits_to_f64(v).reshape(v.shape)
        X = f(x).reshape(-1, K)
        refs.append(oracle.linear_fwd(Wd, X, f(A), f(B), 16.0).reshape((m, N) if m > 1 else (N,)))
    ys = ops.gemv(jobs)
    torch.cuda.synchronize()
    for i, (y, ref) in enumerate(zip(ys, refs)):
        assert_close(torch_to_f64(y), ref, f"decode m{m} job {i}")


def test_mixed_formats_in_one_gemv_call_are_rejected():
    wb = _weights("normal", 64, 128, 7)
    x = bits_to_torch(synth.to_bf16_bits(np.ones(128, dtype=np.float32)))
    W = bits_to_torch(wb)
    jobs = [ops.GemvJob(ops.quantize(W, absmax_format="linear"), x), ops.GemvJob(ops.quantize(W, absmax_format="fp8"), x)]
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        ops.gemv(jobs)
