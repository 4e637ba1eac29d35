"""GPU parity of the layer-set group calls (qlora_group_fwd / _bwd) against
the fp64 group oracle (oracle/group.py), and against the per-linear calls.

Per linear, Y_g, U_g, dA_g and dB_g must equal those of qlora_linear_fwd /
_bwd on the staged path bit for bit (same products, same accumulation
order); dX, which sums the G linears inside one product, and every output at
M < 1024 (where the per-linear calls take the fused path) are held to the
oracle tolerances of tests/helpers.py.  Shapes put group boundaries inside
the dense product's 128/192/256-row tiles and leave ragged token tails.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_nf4_amd import ops, synth
from tests.helpers import assert_close, bits_to_torch, torch_to_bits, torch_to_f64

pytestmark = pytest.mark.gpu


def _draw(G, M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    g = lambda shape, std: synth.to_bf16_bits(rng.standard_normal(shape) * std)
    Ws = [g((N, K), 0.02) for _ in range(G)]
    return dict(Ws=Ws, X=g((M, K), 1.0), dY=g((M, G * N), 1.0),
                A=g((G * r, K), 0.01) if r else None, B=g((G * N, r), 0.01) if r else None)


def _oracle_deq(bits, codebook, fmt):
    c, a, s = oracle.quantize(bits, codebook, fmt)
    return oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, bits.size, codebook, fmt)).reshape(bits.shape)


def _check(G, M, N, K, r, seed, alpha=16.0, codebooks=None, formats=None):
    label = f"G={G} M={M} N={N} K={K} r={r}"
    print(f"[group parity] {label}", flush=True)
    codebooks = codebooks or ["nf4"] * G
    formats = formats or ["linear"] * G
    d = _draw(G, M, N, K, r, seed)
    qs = [ops.quantize(bits_to_torch(W), codebook=cb, absmax_format=f) for W, cb, f in zip(d["Ws"], codebooks, formats)]
    X, dY = bits_to_torch(d["X"]), bits_to_torch(d["dY"])
    A = bits_to_torch(d["A"]) if r else None
    B = bits_to_torch(d["B"]) if r else None
    if r:
        Y, U = ops.group_fwd(qs, X, A, B, alpha, save_u=True)
    else:
        Y, U = ops.group_fwd(qs, X), None
    dX, dA, dB = ops.group_bwd(qs, X, dY, A, B, alpha, U=U)
    # U recomputed inside the backward: the same bits
    dX2, dA2, dB2 = ops.group_bwd(qs, X, dY, A, B, alpha)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2)
    if r:
        assert torch.equal(dA, dA2) and torch.equal(dB, dB2)

    Wds = [_oracle_deq(W, cb, f) for W, cb, f in zip(d["Ws"], codebooks, formats)]
    f64 = lambda k: None if d[k] is None else oracle.bf16_bits_to_f64(d[k]).reshape(d[k].shape)
    Xr, Ar, Br, dYr = f64("X"), f64("A"), f64("B"), f64("dY")
    Yr = oracle.group_fwd(Wds, Xr, Ar, Br, alpha)
    dXr, dAr, dBr = oracle.group_bwd(Wds, Xr, dYr, Ar, Br, alpha)
    assert_close(torch_to_f64(Y), Yr, f"{label} Y")
    assert_close(torch_to_f64(dX), dXr, f"{label} dX")
    if r:
        assert_close(torch_to_f64(U), Xr @ Ar.T, f"{label} U")
        assert_close(torch_to_f64(dA), dAr, f"{label} dA")
        assert_close(torch_to_f64(dB), dBr, f"{label} dB")
    return dict(qs=qs, X=X, dY=dY, A=A, B=B, Y=Y, U=U, dX=dX, dA=dA, dB=dB)


@pytest.mark.parametrize("G,M,N,K,r", [
    (3, 300, 320, 192, 16),     # q/k/v-like; boundaries at rows 320, 640 inside tiles
    (2, 257, 512, 256, 64),     # gate/up-like; one token past a tile
    (4, 129, 128, 128, 64),     # G r = 256, the largest combined rank
    (3, 1, 64, 64, 8),          # one token, smallest shapes
    (1, 200, 448, 128, 32),     # a group of one
])
def test_group_matches_oracle(G, M, N, K, r):
    _check(G, M, N, K, r, seed=G * 1000 + M)


def test_group_without_adapters():
    _check(3, 140, 192, 128, 0, seed=5)


def test_group_mixed_codebooks_and_formats():
    # every weight keeps its own codebook and second-level format
    _check(3, 96, 256, 192, 16, seed=6, codebooks=["nf4", "fp4", "int4"], formats=["linear", "fp8", "fp8"])


@pytest.mark.parametrize("G,M,N,K,r", [
    (3, 1100, 320, 256, 64),    # the per-linear calls take the staged path from 1024 tokens
    (2, 1024, 704, 192, 32),
])
def test_group_equals_per_linear_staged_calls(G, M, N, K, r):
    out = _check(G, M, N, K, r, seed=G * 7 + M)
    qs, X, dY, A, B = out["qs"], out["X"], out["dY"], out["A"], out["B"]
    alpha = 16.0
    for g in range(G):
        Ag, Bg = A[g * r:(g + 1) * r].contiguous(), B[g * N:(g + 1) * N].contiguous()
        dYg = dY[:, g * N:(g + 1) * N].contiguous()
        Yg, Ug = ops.linear_fwd(qs[g], X, Ag, Bg, alpha, save_u=True)
        _, dAg, dBg = ops.linear_bwd(qs[g], X, dYg, Ag, Bg, alpha, U=Ug, need_dx=False)
        torch.cuda.synchronize()
        assert torch.equal(out["Y"][:, g * N:(g + 1) * N], Yg), f"Y_{g}"
        assert torch.equal(out["U"][:, g * r:(g + 1) * r], Ug), f"U_{g}"
        assert torch.equal(out["dA"][g * r:(g + 1) * r], dAg), f"dA_{g}"
        assert torch.equal(out["dB"][g * N:(g + 1) * N], dBg), f"dB_{g}"


def _rows(M, n, seed):
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], inner]))


# the groups of the layer sets bench.py times: q/k/v and gate/up
FULL = [("llama7b", (0, 1, 2)), ("llama7b", (4, 5)), ("llama65b", (0, 1, 2))]
SET_INDEX = {"llama7b": 1, "llama13b": 2, "llama65b": 3}


@pytest.mark.parametrize("set_name,idx", FULL)
def test_group_full_shape(set_name, idx):
    """The full layer-set shapes, built as bench.py builds them: the group's X
    is the first linear's, dY and the adapters are the linears' own, side by
    side.  Y and dX on sampled token rows against the oracle (every column),
    dA and dB in full; Y_g, dA_g, dB_g bitwise against the per-linear calls."""
    cfg = synth.LAYER_SETS[set_name]
    M, r, alpha = cfg["M"], cfg["r"], cfg["alpha"]
    names = [cfg["linears"][i][0] for i in idx]
    _, N, K = cfg["linears"][idx[0]]
    G = len(idx)
    label = f"{set_name} {'/'.join(names)} G={G} {N}x{K} M={M}"
    print(f"[group full-size] {label}", flush=True)
    ts = [synth.linear_inputs(N, K, M, r, synth.layer_set_seed(SET_INDEX[set_name], i), "cuda",
                              outliers=cfg["outliers"]) for i in idx]
    X = ts[0]["X"]
    A = torch.cat([t["A"] for t in ts]).contiguous()
    B = torch.cat([t["B"] for t in ts]).contiguous()
    dY = torch.cat([t["dY"] for t in ts], dim=1).contiguous()
    qs = [ops.quantize(t["W"]) for t in ts]
    Y, U = ops.group_fwd(qs, X, A, B, alpha, save_u=True)
    dX, dA, dB = ops.group_bwd(qs, X, dY, A, B, alpha, U=U)
    torch.cuda.synchronize()
    for g, t in enumerate(ts):
        Yg, Ug = ops.linear_fwd(qs[g], X, t["A"], t["B"], alpha, save_u=True)
        _, dAg, dBg = ops.linear_bwd(qs[g], X, t["dY"], t["A"], t["B"], alpha, U=Ug, need_dx=False)
        torch.cuda.synchronize()
        assert torch.equal(Y[:, g * N:(g + 1) * N], Yg), f"{label}: Y_{g}"
        assert torch.equal(dA[g * r:(g + 1) * r], dAg), f"{label}: dA_{g}"
        assert torch.equal(dB[g * N:(g + 1) * N], dBg), f"{label}: dB_{g}"
        del Yg, Ug, dAg, dBg

    Wds = []
    for t in ts:
        w = torch_to_bits(t["W"]).ravel()
        c, a, s = oracle.quantize(w)
        Wds.append(oracle.bf16_bits_to_f64(oracle.dequant(c, a, s, w.size)).reshape(N, K))
    Xr, Ar, Br, dYr = (torch_to_f64(v) for v in (X, A, B, dY))
    rows = _rows(M, 32, N + K + G)
    assert_close(torch_to_f64(Y)[rows], oracle.group_fwd(Wds, Xr[rows], Ar, Br, alpha), f"{label} Y (32 rows)")
    dXr, _, _ = oracle.group_bwd(Wds, Xr[rows], dYr[rows], Ar, Br, alpha)
    assert_close(torch_to_f64(dX)[rows], dXr, f"{label} dX (32 rows)")
    for g in range(G):   # dA_g, dB_g do not involve the weights
        dAr, dBr = oracle.adapter_grads(Xr, dYr[:, g * N:(g + 1) * N], Ar[g * r:(g + 1) * r],
                                        Br[g * N:(g + 1) * N], alpha)
        assert_close(torch_to_f64(dA[g * r:(g + 1) * r]), dAr, f"{label} dA_{g}")
        assert_close(torch_to_f64(dB[g * N:(g + 1) * N]), dBr, f"{label} dB_{g}")


@pytest.mark.parametrize("G,M,N,K,r", [(3, 300, 320, 192, 16), (2, 1100, 256, 256, 64)])
def test_building_blocks_compose_to_the_group_calls(G, M, N, K, r):
    """lora_down (stacked A) + group_dequant + bf16_group_fwd is group_fwd, and
    group_lora_dy_b + group_dequant_t + bf16_group_dx + group_lora_grads is
    group_bwd, bit for bit (the same kernels in the same order)."""
    print(f"[group building blocks] G={G} M={M} N={N} K={K} r={r}", flush=True)
    d = _draw(G, M, N, K, r, seed=99 + G)
    qs = [ops.quantize(bits_to_torch(W)) for W in d["Ws"]]
    X, dY, A, B = (bits_to_torch(d[k]) for k in ("X", "dY", "A", "B"))
    alpha = 16.0
    Y, U = ops.group_fwd(qs, X, A, B, alpha, save_u=True)
    dX, dA, dB = ops.group_bwd(qs, X, dY, A, B, alpha, U=U)

    U2 = ops.lora_down(X, A)
    Y2 = ops.bf16_group_fwd(ops.group_dequant(qs), G, X, U2, B, alpha)
    Gm = ops.group_lora_dy_b(dY, B, G)
    dX2 = ops.bf16_group_dx(ops.group_dequant(qs, transposed=True), G, dY, Gm, A, alpha)
    dA2, dB2 = ops.group_lora_grads(X, dY, U2, Gm, G, alpha)
    torch.cuda.synchronize()
    for name, a, b in (("U", U, U2), ("Y", Y, Y2), ("dX", dX, dX2), ("dA", dA, dA2), ("dB", dB, dB2)):
        assert torch.equal(a, b), name
    # the stacks are the per-weight dequantizations, in place
    Wd, WdT = ops.group_dequant(qs), ops.group_dequant(qs, transposed=True)
    for g, q in enumerate(qs):
        assert torch.equal(Wd[g * N:(g + 1) * N], ops.dequant(q))
        assert torch.equal(WdT[:, g * N:(g + 1) * N], ops.dequant_t(q))


def test_group_dequant_mixed_formats_and_long_groups():
    """The group dequantization batches consecutive weights of one codebook
    and absmax format into one launch (at most eight): a group that mixes
    formats, and one longer than a launch holds, still gives every weight's
    own dequantization in its place, bit for bit."""
    print("[group dequant] mixed codebooks / formats, G = 3 and G = 11", flush=True)
    N, K = 128, 320
    fmts = [("nf4", "linear"), ("fp4", "linear"), ("nf4", "fp8")]
    for G, pick in ((3, lambda g: fmts[g]), (11, lambda g: fmts[0] if g != 9 else fmts[2])):
        Ws = [synth.normal_bf16((N, K), 0.02, 700 + 17 * G + g, "cuda") for g in range(G)]
        qs = [ops.quantize(W, codebook=pick(g)[0], absmax_format=pick(g)[1]) for g, W in enumerate(Ws)]
        Wd, WdT = ops.group_dequant(qs), ops.group_dequant(qs, transposed=True)
        torch.cuda.synchronize()
        for g, q in enumerate(qs):
            assert torch.equal(Wd[g * N:(g + 1) * N], ops.dequant(q)), (G, g)
            assert torch.equal(WdT[:, g * N:(g + 1) * N], ops.dequant_t(q)), (G, g)


def test_group_dequant_past_the_last_level_cache_equals_per_weight():
    """A launch whose bf16 output exceeds 256 MB (the last-level cache) runs
    its workgroups in reverse order; each weight alone here is below that
    size and runs in order.  Both must give the same bits: the three 65B
    q/k/v weights (403 MB stacked, 134 MB each), ragged row count on a
    fourth group (3 x 8200 rows, so the reversed grid's first workgroup is a
    partial one)."""
    for N, K in ((8192, 8192), (8200, 8192)):
        print(f"[group dequant] reversed order, 3 x {N} x {K}", flush=True)
        qs = [ops.quantize(synth.normal_bf16((N, K), 0.02, 900 + g, "cuda", outliers=0.001)) for g in range(3)]
        assert 3 * N * K * 2 > (256 << 20) and N * K * 2 < (256 << 20)
        Wd = ops.group_dequant(qs)
        for g, q in enumerate(qs):
            assert torch.equal(Wd[g * N:(g + 1) * N], ops.dequant(q)), g
        del Wd
        WdT = ops.group_dequant(qs, transposed=True)
        for g, q in enumerate(qs):
            assert torch.equal(WdT[:, g * N:(g + 1) * N], ops.dequant_t(q)), g
        del WdT, qs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
