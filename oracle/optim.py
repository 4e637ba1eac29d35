"""The optimizer step on the LoRA matrices (the step after the backward).

The pages name paged optimizers, whose states move between GPU and CPU
memory (glossary page, "Definition"; deepfa.ir "3. Paged Optimizers"), but
not the optimizer.  Reading R17: AdamW (Adam with decoupled weight decay and
bias correction) on fp32 master values of A and B, with fp32 moment
estimates and the fp32 gradients dA, dB of the backward pass; after the step
the bf16 copies the layer reads are refreshed by round-to-nearest-even.
For step t >= 1:

  m <- b1 m + (1 - b1) g
  v <- b2 v + (1 - b2) g^2
  p <- p - lr * ( (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps) + wd * p )

This function is the definition in fp64.
"""

import numpy as np


def adamw_step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, t):
    """One AdamW step in fp64; returns the new (p, m, v)."""
    p, g, m, v = (np.asarray(a, dtype=np.float64) for a in (p, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** t)
    vh = v / (1.0 - beta2 ** t)
    p = p - lr * (mh / (np.sqrt(vh) + eps) + weight_decay * p)
    return p, m, v
