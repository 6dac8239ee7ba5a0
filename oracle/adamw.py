"""Oracle: one AdamW step on the adapter parameters, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages keep optimizer state only for the adapters, in fp32, and page it between
GPU and CPU memory ([Explainer] "Paged optimizers"; [Glossary] "Optimizer States");
the optimizer is Adam with decoupled weight decay (AdamW; [Addaly] names
paged_adamw_8bit, [Glossary] "like AdamW").  The pages do not write the update out;
this is the standard decoupled-weight-decay Adam step with bias correction:

    p <- p (1 - lr wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

computed here in float64 with no intermediate rounding.
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, t: int, lr: float, b1: float = 0.9, b2: float = 0.999, eps: float = 1e-8,
               wd: float = 0.0):
    """Returns the new (p, m, v) as float64 arrays; t >= 1 is the step number."""
    p = np.asarray(p, np.float64) * (1.0 - lr * wd)
    g = np.asarray(g, np.float64)
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v
