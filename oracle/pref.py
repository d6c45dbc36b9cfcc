"""Preference-loss heads on one (chosen, rejected) pair -- oracle side.

Test infrastructure only (see ``oracle/__init__``).  The pages list DPO,
ORPO, SimPO and KTO as the preference methods that run on the layer stream,
and state that KTO uses the same adapters-disabled reference as DPO (page
"Soup ... radar note", section "In detail"); they give no formulas.  Each head
below follows the loss as its own paper defines it, in float64, as a function
of the sequence log-likelihoods the stream produces:

  pi_x  = sum over response tokens t of log p_theta(y_t | y_<t), x in {c, r}
  rho_x = the same with the adapters disabled (DPO, KTO only)
  n_x   = number of response tokens

and returns the loss and dL/dpi_c, dL/dpi_r (the references carry no
gradient).  sigma is the logistic function, softplus(a) = log(1 + e^a).

  dpo    Rafailov et al. 2023, sigmoid loss:
           z = beta((pi_c - rho_c) - (pi_r - rho_r)),  L = softplus(-z)
  simpo  Meng et al. 2024, length-normalised, reference-free, target margin:
           z = beta pi_c / n_c - beta pi_r / n_r - gamma,  L = softplus(-z)
  orpo   Hong et al. 2024, SFT on the chosen response plus odds ratio:
           l_x = pi_x / n_x,  logodds_x = l_x - log(1 - e^{l_x}),
           L = -l_c + lam softplus(-(logodds_c - logodds_r))
  kto    Ethayarajh et al. 2024, chosen desirable, rejected undesirable:
           r_x = pi_x - rho_x,  z0 = max(0, (r_c + r_r) / 2) (no gradient),
           L = (lam_d (1 - sigma(beta (r_c - z0))) + lam_u (1 - sigma(beta (z0 - r_r)))) / 2
         Reading: the paper's reference point z0 is a KL estimate from
         mismatched (prompt, completion) pairs of a batch; a single pair that
         shares its prompt has none, so z0 is the batch mean of the log
         ratios, clamped at zero and held constant, and the loss is the mean
         over the two examples.
"""
from __future__ import annotations

import math

KINDS = ("dpo", "simpo", "orpo", "kto")
# Defaults of the respective papers' reference recipes.
DEFAULTS = {"beta": {"dpo": 0.1, "simpo": 2.0, "orpo": 0.0, "kto": 0.1},
            "gamma": 1.0, "lam": 0.1, "lam_d": 1.0, "lam_u": 1.0}


def sigmoid(a: float) -> float:
    if a >= 0:
        return 1.0 / (1.0 + math.exp(-a))
    e = math.exp(a)
    return e / (1.0 + e)


def softplus(a: float) -> float:
    return max(a, 0.0) + math.log1p(math.exp(-abs(a)))


def kto_z0(pi, ref) -> float:
    return max(0.0, 0.5 * ((pi[0] - ref[0]) + (pi[1] - ref[1])))


def head(kind, pi, ref, n, beta=None, gamma=1.0, lam=0.1, lam_d=1.0, lam_u=1.0, z0=None):
    """Loss and (dL/dpi_c, dL/dpi_r) of preference head ``kind``.

    pi, ref, n: (chosen, rejected) pairs; ref is ignored by simpo and orpo.
    z0 (kto only): reference point to hold fixed; default kto_z0(pi, ref)."""
    if kind not in KINDS:
        raise ValueError(kind)
    pc, pr = float(pi[0]), float(pi[1])
    nc, nr = float(n[0]), float(n[1])
    if beta is None:
        beta = DEFAULTS["beta"][kind]
    if kind == "dpo":
        z = beta * ((pc - ref[0]) - (pr - ref[1]))
        s = sigmoid(-z)
        return softplus(-z), (-beta * s, beta * s)
    if kind == "simpo":
        z = beta * pc / nc - beta * pr / nr - gamma
        s = sigmoid(-z)
        return softplus(-z), (-beta * s / nc, beta * s / nr)
    if kind == "orpo":
        lc, lr = pc / nc, pr / nr
        qc, qr = -math.expm1(lc), -math.expm1(lr)          # 1 - p_x, p_x = e^{l_x}
        rr = (lc - math.log(qc)) - (lr - math.log(qr))
        s = sigmoid(-rr)
        # d logodds / d l = 1 / (1 - p)
        return -lc + lam * softplus(-rr), ((-1.0 - lam * s / qc) / nc, (lam * s / qr) / nr)
    # kto
    if z0 is None:
        z0 = kto_z0(pi, ref)
    u = beta * ((pc - ref[0]) - z0)
    v = beta * (z0 - (pr - ref[1]))
    su, sv = sigmoid(u), sigmoid(v)
    loss = 0.5 * (lam_d * (1.0 - su) + lam_u * (1.0 - sv))
    return loss, (-0.5 * lam_d * beta * su * (1.0 - su), 0.5 * lam_u * beta * sv * (1.0 - sv))


def needs_reference(kind) -> bool:
    return kind in ("dpo", "kto")
