"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and casts them to bfloat16; it holds
none of the method's arithmetic.  The shapes stand in for the LLaMA
finetunes the pages describe (glossary page "Definition": LLaMA 7B-65B;
deepfa.ir "Optimization Tips": LoRA on the attention projections, rank 8-64);
no real weights or data are used.

Distributions (reading R14): "N(0, 0.02)" is a normal with standard
deviation 0.02; "0.1% outliers x8" is an independent Bernoulli(0.001) mask
whose weights are multiplied by 8 before the bf16 cast.
"""

import numpy as np
import torch

# (name, N = out features, K = in features) of one transformer layer's linears
def _layer(d, f):
    return [("q", d, d), ("k", d, d), ("v", d, d), ("o", d, d),
            ("gate", f, d), ("up", f, d), ("down", d, f)]


LAYER_SETS = {
    "small": dict(linears=[("w", 1024, 1024)], M=256, r=8, alpha=16.0, outliers=0.0),
    "llama7b": dict(linears=_layer(4096, 11008), M=2048, r=64, alpha=16.0, outliers=0.0),
    "llama13b": dict(linears=_layer(5120, 13824), M=2048, r=64, alpha=16.0, outliers=0.0),
    "llama65b": dict(linears=_layer(8192, 22016), M=4096, r=64, alpha=16.0, outliers=0.001),
}
DECODE_LAYERS = 80


def small_numpy(seed=0):
    """The 1024x1024 single-linear case, drawn with numpy in a fixed order.

    Order W, A, B, X, dY; each drawn in fp64, scaled, cast to fp32 and then
    to bf16 (round to nearest even).  Returns uint16 bit patterns.
    """
    rng = np.random.default_rng(seed)
    N = K = 1024
    M, r = 256, 8
    out = {}
    for name, shape, std in (("W", (N, K), 0.02), ("A", (r, K), 0.01), ("B", (N, r), 0.01),
                             ("X", (M, K), 1.0), ("dY", (M, N), 1.0)):
        v = (rng.standard_normal(shape) * std).astype(np.float32)
        out[name] = to_bf16_bits(v)
    out.update(M=M, N=N, K=K, r=r, alpha=16.0)
    return out


def to_bf16_bits(a):
    """fp32 numpy array -> bf16 bit patterns (uint16) via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, std, seed, device, outliers=0.0, gen_dtype=torch.float32):
    """A bf16 tensor ~N(0, std), optionally with x8 outliers, from a seeded generator."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=gen_dtype)
    t.mul_(std)
    if outliers > 0:
        mask = torch.rand(shape, generator=g, device=device) < outliers
        t[mask] *= 8.0
    return t.to(torch.bfloat16)


def linear_inputs(N, K, M, r, seed, device, outliers=0.0, with_grad=True):
    """Inputs of one QLoRA linear: W [N,K], A [r,K], B [N,r], X [M,K], dY [M,N]."""
    base = int(seed) * 16
    d = dict(
        W=normal_bf16((N, K), 0.02, base + 0, device, outliers),
        A=normal_bf16((r, K), 0.01, base + 1, device),
        B=normal_bf16((N, r), 0.01, base + 2, device),
        X=normal_bf16((M, K), 1.0, base + 3, device),
    )
    if with_grad:
        d["dY"] = normal_bf16((M, N), 1.0, base + 4, device)
    return d


def layer_set_seed(set_index, linear_index, layer=0):
    """Seed rule: 1000 * (layer or set) + linear index."""
    return 1000 * (layer if layer else set_index) + linear_index
