"""GPU parity of the dense bf16 GEMM on a dequantized weight (qlora_dequant
followed by qlora_bf16_fwd) against the fp64 oracle.

Y = X deq(W)^T + s (X A^T) B^T within the forward tolerances, on shapes that
span several 256 x 256 tiles with ragged edges, r = 0, a LoRA-dominant case,
and the largest rank.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_f64

pytestmark = pytest.mark.gpu


def _case(N, K, M, r, seed, ab_std=0.01, w_std=0.02):
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    W = g((N, K), w_std) if w_std else np.zeros((N, K), dtype=np.uint16)
    return dict(W=W, X=g((M, K), 1.0), A=g((r, K), ab_std) if r else None, B=g((N, r), ab_std) if r else None,
                alpha=16.0)


def _oracle(d):
    c, a, s = oracle.quantize(d["W"])
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size)).reshape(d["W"].shape)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    return Wd, oracle.linear_fwd(Wd, f("X"), f("A"), f("B"), d["alpha"])


@pytest.mark.parametrize("N,K,M,r", [(1024, 1024, 256, 8), (1000, 576, 300, 16), (264, 8192, 520, 64),
                                     (512, 1088, 777, 0), (768, 2048, 1024, 128), (8, 64, 1, 8)])
def test_dense_forward_matches_oracle(N, K, M, r):
    d = _case(N, K, M, r, seed=N + K + M + r)
    print(f"[dense parity] N{N} K{K} M{M} r{r}", flush=True)
    q = ops.quantize(bits_to_torch(d["W"]))
    Wd = ops.dequant(q)
    X = bits_to_torch(d["X"])
    U = ops.lora_down(X, bits_to_torch(d["A"])) if r else None
    Y = ops.bf16_fwd(Wd, X, U, bits_to_torch(d["B"]) if r else None, d["alpha"])
    torch.cuda.synchronize()
    Wref, Yref = _oracle(d)
    assert np.array_equal(torch_to_f64(Wd), Wref)   # the dequantized weight is bit-exact
    assert_close(torch_to_f64(Y), Yref, f"Y N{N} K{K} M{M} r{r}")


@pytest.mark.parametrize("w_std,ab_std", [(0.0, 1.0), (0.02, 1.0)])
def test_dense_forward_lora_stress(w_std, ab_std):
    # W = 0 (pure LoRA) and a LoRA-dominant case: the tail cannot hide
    d = _case(520, 1024, 600, 64, seed=77, ab_std=ab_std, w_std=w_std)
    q = ops.quantize(bits_to_torch(d["W"]))
    X = bits_to_torch(d["X"])
    U = ops.lora_down(X, bits_to_torch(d["A"]))
    Y = ops.bf16_fwd(ops.dequant(q), X, U, bits_to_torch(d["B"]), d["alpha"])
    torch.cuda.synchronize()
    assert_close(torch_to_f64(Y), _oracle(d)[1], f"stress w{w_std} ab{ab_std}")


@pytest.mark.parametrize("N,K,M,r", [(1024, 1024, 256, 8), (1088, 576, 300, 16), (320, 8192, 520, 128),
                                     (512, 1088, 777, 0), (64, 64, 1, 8)])
def test_dense_dx_matches_oracle(N, K, M, r):
    """qlora_dequant_t then qlora_bf16_dx: dX = dY deq(W) + s (dY B) A."""
    rng = np.random.default_rng(N + K + M + r + 1)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    d = dict(W=g((N, K), 0.02), dY=g((M, N), 1.0), A=g((r, K), 0.2) if r else None,
             B=g((N, r), 0.2) if r else None, alpha=16.0)
    print(f"[dense dX parity] N{N} K{K} M{M} r{r}", flush=True)
    q = ops.quantize(bits_to_torch(d["W"]))
    dY = bits_to_torch(d["dY"])
    A = bits_to_torch(d["A"]) if r else None
    G = ops.lora_dy_b(dY, bits_to_torch(d["B"])) if r else None
    dX = ops.bf16_dx(ops.dequant_t(q), dY, G, A, d["alpha"])
    torch.cuda.synchronize()
    c, a, s = oracle.quantize(d["W"])
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size)).reshape(N, K)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    dXr = f("dY") @ Wd
    if r:
        dXr = dXr + d["alpha"] / r * (f("dY") @ f("B")) @ f("A")
    assert_close(torch_to_f64(dX), dXr, f"dX N{N} K{K} M{M} r{r}")


# Tile widths: on 256 CUs, (5120 rows, 2048 tokens) runs 192-row tiles in one
# round; (4352 rows, 4096 tokens) fills one round of 256-row tiles and runs
# the last 256 rows as 128-row tiles in a second launch; small shapes run
# 128-row tiles.  Forward (weight rows = N) and dX (output columns = K).
@pytest.mark.parametrize("N,K,M", [(5120, 128, 2048), (4352, 128, 4096), (320, 512, 300)])
def test_dense_forward_tile_widths(N, K, M):
    r = 16
    d = _case(N, K, M, r, seed=N + 2 * K + M, ab_std=0.2)
    print(f"[dense widths] fwd N{N} K{K} M{M}", flush=True)
    q = ops.quantize(bits_to_torch(d["W"]))
    X = bits_to_torch(d["X"])
    U = ops.lora_down(X, bits_to_torch(d["A"]))
    Y = ops.bf16_fwd(ops.dequant(q), X, U, bits_to_torch(d["B"]), d["alpha"])
    torch.cuda.synchronize()
    assert_close(torch_to_f64(Y), _oracle(d)[1], f"Y N{N} K{K} M{M}")


@pytest.mark.parametrize("N,K,M", [(128, 5120, 2048), (128, 4352, 4096)])
def test_dense_dx_tile_widths(N, K, M):
    test_dense_dx_matches_oracle(N, K, M, 16)


# Split contraction: dX products with at most 128 output tiles of 256 x 256
# and a contraction of 16384 columns or more run the contraction in two
# halves and add the fp32 partials (the 7B gate/up dX has 128 tiles over
# 22016 columns).  Ragged tokens (300) and output columns (576 = two and a
# quarter tiles), the LoRA tail (split 0 only) large enough to show.
@pytest.mark.parametrize("N,K,M,r", [(16384, 576, 300, 32), (16448, 512, 256, 0), (22016, 256, 64, 64)])
def test_dense_dx_split_contraction(N, K, M, r):
    rng = np.random.default_rng(N + K + M + r + 5)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    d = dict(W=g((N, K), 0.02), dY=g((M, N), 1.0), A=g((r, K), 0.5) if r else None,
             B=g((N, r), 0.5) if r else None, alpha=16.0)
    from bit_quantized_finetuning_nf4_amd import _lib
    split_bytes = ops.workspace_bytes(_lib.QLORA_OP_BF16_DX, M, N, K, r, 1)
    print(f"[dense dX split] N{N} K{K} M{M} r{r} split workspace {split_bytes}", flush=True)
    assert split_bytes == 2 * M * K * 4
    q = ops.quantize(bits_to_torch(d["W"]))
    dY = bits_to_torch(d["dY"])
    A = bits_to_torch(d["A"]) if r else None
    G = ops.lora_dy_b(dY, bits_to_torch(d["B"])) if r else None
    WdT = ops.dequant_t(q)
    dX = ops.bf16_dx(WdT, dY, G, A, d["alpha"])                      # split (workspace allocated)
    small = torch.empty(256, dtype=torch.uint8, device=dY.device)   # too small: unsplit
    dX1 = ops.bf16_dx(WdT, dY, G, A, d["alpha"], ws=small)
    torch.cuda.synchronize()
    c, a, s = oracle.quantize(d["W"])
    Wd = oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, d["W"].size)).reshape(N, K)
    f = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    dXr = f("dY") @ Wd
    if r:
        dXr = dXr + d["alpha"] / r * (f("dY") @ f("B")) @ f("A")
    assert_close(torch_to_f64(dX), dXr, f"split dX N{N} K{K} M{M} r{r}")
    assert_close(torch_to_f64(dX1), dXr, f"unsplit dX N{N} K{K} M{M} r{r}")
    # the two orders of summation differ by rounding only
    diff = (dX.float() - dX1.float()).abs().max().item()
    assert diff <= 2e-2 * dX1.float().abs().max().item()
