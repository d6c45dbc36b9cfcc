"""AdamW on the LoRA parameters -- oracle side (test infrastructure only).

The pages train with a learning rate of 2e-5 for 3 epochs (page "Fine tune an
8B model on a 4GB laptop GPU (Soup setup)", section "Step 1, the config") and
propose 20 streamed against 20 resident steps with matching loss curves as the
practical check (page "Fine-Tune an 8B Model on a 4GB Laptop GPU: Hands-On
Guide", section "The gotchas nobody's mentioning yet").  They do not name the
optimizer; the reading taken here is AdamW with decoupled weight decay (the usual LoRA
fine-tuning optimizer), betas (0.9, 0.999), eps 1e-8, weight decay 0 unless
given, applied to every A and B entry of the packed float32 LoRA vector:

    p <- p * (1 - lr * wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)

``Prec("fp64")`` runs it in float64; ``Prec("mirror")`` in float32 with the two
bias-correction factors computed in float64 and rounded once, as the device
kernel does.
"""
from __future__ import annotations

import numpy as np


def adamw_step(P, p, g, m, v, t, lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """One update at step t (1-based).  Returns new (p, m, v) in P's dtype."""
    dt = P.dt
    p, g, m, v = (np.asarray(x, dtype=dt) for x in (p, g, m, v))
    step_size = dt(lr / (1.0 - b1 ** t))
    inv_sqrt_bc2 = dt(1.0 / np.sqrt(1.0 - b2 ** t))
    p = p * dt(1.0 - lr * wd)
    m = dt(b1) * m + dt(1.0 - b1) * g
    v = dt(b2) * v + dt(1.0 - b2) * (g * g)
    denom = np.sqrt(v) * inv_sqrt_bc2 + dt(eps)
    p = p - step_size * (m / denom)
    return p.astype(dt), m.astype(dt), v.astype(dt)
