"""A group of LoRA linears that read one input, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

LoRA is applied to several linears of each transformer layer (deepfa.ir blog,
"Optimization Tips", target modules), and in a LLaMA layer some of them read
the same input: the query, key and value projections read the normalised
hidden state, the gate and up projections the second normalised state.

Reading R20 (the pages do not treat such groups): a group is G independent
linears of the layer in "linear.py", each with its own dequantized weight
Wd_g [N x K], adapter (A_g [r x K], B_g [N x r]) and the shared alpha,
applied to one X [M x K].  With the adapters stacked, A = [A_0; A_1; ..]
[G r x K] and B = [B_0; B_1; ..] [G N x r], and the outputs side by side:

    Y = [Y_0 | Y_1 | ..]           Y_g = linear_fwd(Wd_g, X, A_g, B_g)
    dY = [dY_0 | dY_1 | ..]        (the upstream gradient of Y)
    dX = sum_g dX_g                (X feeds every linear of the group)
    dA = [dA_0; dA_1; ..], dB = [dB_0; dB_1; ..]

Each output is the per-linear definition; nothing is fused here.
"""

import numpy as np

from .linear import linear_bwd, linear_fwd


def _split(a, G, axis):
    return None if a is None else np.split(np.asarray(a, dtype=np.float64), G, axis=axis)


def group_fwd(Wds, X, A=None, B=None, alpha=0.0):
    """Y [M x G N] for weights Wds (G of [N x K]) and stacked adapters."""
    G = len(Wds)
    As, Bs = _split(A, G, 0), _split(B, G, 0)
    outs = [linear_fwd(Wds[g], X, None if As is None else As[g], None if Bs is None else Bs[g], alpha)
            for g in range(G)]
    return np.concatenate(outs, axis=1)


def group_bwd(Wds, X, dY, A=None, B=None, alpha=0.0):
    """(dX [M x K], dA [G r x K] or None, dB [G N x r] or None)."""
    G = len(Wds)
    As, Bs, dYs = _split(A, G, 0), _split(B, G, 0), _split(dY, G, 1)
    dX, dA, dB = None, [], []
    for g in range(G):
        dXg, dAg, dBg = linear_bwd(Wds[g], X, dYs[g], None if As is None else As[g],
                                   None if Bs is None else Bs[g], alpha)
        dX = dXg if dX is None else dX + dXg
        dA.append(dAg)
        dB.append(dBg)
    if As is None:
        return dX, None, None
    return dX, np.concatenate(dA, axis=0), np.concatenate(dB, axis=0)
