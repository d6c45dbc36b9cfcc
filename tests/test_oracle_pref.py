"""Pins of the oracle's preference heads (oracle.pref) and of the preference
step around them (oracle.model.pref_step).

The pages name DPO, ORPO, SimPO and KTO without formulas; each head follows its
paper.  They are pinned by closed forms at the points where the sigmoid term
is exactly 1/2, by an expression of ORPO's odds through p / (1 - p) directly,
by float64 central differences of every head and of the whole step with
respect to LoRA entries, by exact cancellation when chosen == rejected, and by
the step's DPO head agreeing with the separately pinned DPO step."""
import math

import numpy as np
import pytest

import synth
from oracle import model as om
from oracle import pref
from tests.helpers import MICRO, oracle_model

P64 = om.Prec("fp64")
PM = om.Prec("mirror")
LN2 = math.log(2.0)


def test_closed_forms_at_the_midpoint():
    n = (40, 40)
    loss, g = pref.head("dpo", (-50.0, -60.0), (-55.0, -65.0), n, beta=0.1)
    assert loss == pytest.approx(LN2, abs=1e-15) and g == pytest.approx((-0.05, 0.05), abs=1e-15)
    # SimPO: beta pi_c / n_c - beta pi_r / n_r == gamma puts z at 0.
    beta, gamma = 2.0, 1.0
    pr = -80.0
    pc = (gamma + beta * pr / n[1]) * n[0] / beta
    loss, g = pref.head("simpo", (pc, pr), (0, 0), n, beta=beta, gamma=gamma)
    assert loss == pytest.approx(LN2, abs=1e-14)
    assert g == pytest.approx((-beta / 2 / n[0], beta / 2 / n[1]), abs=1e-15)
    # ORPO with equal log-likelihoods: odds ratio 1, L = mean NLL of chosen + lam ln 2.
    loss, _ = pref.head("orpo", (-30.0, -30.0), (0, 0), n, lam=0.25)
    assert loss == pytest.approx(30.0 / 40 + 0.25 * LN2, abs=1e-14)
    # KTO: policy == reference -> both sigmoids at 1/2, L = (lam_d + lam_u) / 4.
    loss, g = pref.head("kto", (-50.0, -60.0), (-50.0, -60.0), n, beta=0.1, lam_d=1.0, lam_u=1.5)
    assert loss == pytest.approx(2.5 / 4, abs=1e-15)
    assert g == pytest.approx((-0.5 * 0.1 / 4, 0.5 * 1.5 * 0.1 / 4), abs=1e-15)


def test_orpo_odds_by_definition():
    """Log odds from p / (1 - p) with p = exp(mean log-likelihood), written
    without the expm1 form the head uses."""
    n = (10, 7)
    for pc, pr, lam in [(-3.0, -9.0, 0.1), (-12.0, -2.0, 0.5), (-0.5, -0.4, 1.0)]:
        p_c, p_r = math.exp(pc / n[0]), math.exp(pr / n[1])
        ratio = (p_c / (1 - p_c)) / (p_r / (1 - p_r))
        want = -pc / n[0] - lam * math.log(ratio / (1 + ratio))     # -log sigma(log ratio)
        assert pref.head("orpo", (pc, pr), (0, 0), n, lam=lam)[0] == pytest.approx(want, rel=1e-12)


@pytest.mark.parametrize("kind", pref.KINDS)
def test_head_gradients_by_central_differences(kind):
    rng = np.random.default_rng(3)
    h = 1e-6
    for _ in range(25):
        n = (int(rng.integers(5, 60)), int(rng.integers(5, 60)))
        pi = tuple(-rng.uniform(0.2, 8.0) * k for k in n)
        ref = tuple(p + rng.normal(0, 2.0) for p in pi)
        kw = {"beta": float(rng.uniform(0.05, 2.5))}
        if kind == "simpo":
            kw["gamma"] = float(rng.uniform(0, 2))
        if kind == "orpo":
            kw = {"lam": float(rng.uniform(0.05, 1.0))}
        if kind == "kto":
            kw.update(lam_d=float(rng.uniform(0.5, 2)), lam_u=float(rng.uniform(0.5, 2)),
                      z0=pref.kto_z0(pi, ref))              # the reference point is held constant
        _, g = pref.head(kind, pi, ref, n, **kw)
        for i in range(2):
            up, dn = list(pi), list(pi)
            up[i] += h
            dn[i] -= h
            fd = (pref.head(kind, up, ref, n, **kw)[0] - pref.head(kind, dn, ref, n, **kw)[0]) / (2 * h)
            assert fd == pytest.approx(g[i], rel=1e-6, abs=1e-10), (kind, i, pi, ref, n, kw)


def test_kto_reference_point_clamps_at_zero():
    """When the mean log ratio is negative z0 is exactly 0, so holding it
    constant changes nothing and the full loss has the analytic gradient."""
    pi, ref, n = (-50.0, -70.0), (-48.0, -66.0), (30, 30)
    assert pref.kto_z0(pi, ref) == 0.0
    _, g = pref.head("kto", pi, ref, n)
    h = 1e-6
    for i in range(2):
        up, dn = list(pi), list(pi)
        up[i] += h
        dn[i] -= h
        fd = (pref.head("kto", up, ref, n)[0] - pref.head("kto", dn, ref, n)[0]) / (2 * h)
        assert fd == pytest.approx(g[i], rel=1e-6)


def test_step_dpo_head_equals_dpo_step():
    cfg = MICRO
    model = oracle_model(cfg)
    lora = synth.lora_init(cfg, b_std=0.05)
    c, r = synth.dpo_pair(cfg, 12, 4)
    l1, g1, a1 = om.dpo_step(cfg, PM, model, lora, c, r, 4, 0.1)
    l2, g2, a2 = om.pref_step(cfg, PM, model, lora, c, r, 4, "dpo", beta=0.1)
    assert l1 == pytest.approx(l2, rel=1e-12)
    assert np.array_equal(a1["pi"], a2["pi"]) and np.array_equal(a1["ref"], a2["ref"])
    for l in range(cfg.L):
        for nm in om.NAMES:
            for w in range(2):
                np.testing.assert_allclose(g1[l][nm][w], g2[l][nm][w], rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("kind", ["simpo", "orpo", "kto"])
def test_step_gradients_by_central_differences(kind):
    cfg = MICRO
    model = oracle_model(cfg)
    lora = synth.lora_init(cfg, b_std=0.05)
    c, r = synth.dpo_pair(cfg, 12, 4)
    kw = {"simpo": {"beta": 2.0, "gamma": 0.5}, "orpo": {"lam": 0.3}, "kto": {"beta": 0.5}}[kind]
    loss, grads, aux = om.pref_step(cfg, P64, model, lora, c, r, 4, kind, **kw)
    if kind == "kto":
        kw = dict(kw, z0=pref.kto_z0(aux["pi"], aux["ref"]))
    rng = np.random.default_rng(11)
    h = 1e-5
    for _ in range(8):
        l = int(rng.integers(cfg.L)); nm = om.NAMES[int(rng.integers(7))]; w = int(rng.integers(2))
        M = lora[l][nm][w]
        idx = tuple(int(rng.integers(s)) for s in M.shape)
        vals = []
        for sgn in (1, -1):
            lp = [{k: (a.astype(np.float64).copy(), b.astype(np.float64).copy())
                   for k, (a, b) in mods.items()} for mods in lora]
            lp[l][nm][w][idx] += sgn * h
            vals.append(om.pref_step(cfg, P64, model, lp, c, r, 4, kind, **kw)[0])
        fd = (vals[0] - vals[1]) / (2 * h)
        an = grads[l][nm][w][idx]
        assert abs(fd - an) <= 1e-5 * abs(an) + 1e-10, (kind, l, nm, w, fd, an)


def test_identical_pair_cancels():
    """chosen == rejected: SimPO's two terms cancel exactly in every gradient;
    ORPO keeps only its SFT term (the gradients of lam = 0.7 and lam = 0 agree)."""
    cfg = MICRO
    model = oracle_model(cfg)
    lora = synth.lora_init(cfg, b_std=0.05)
    c, _ = synth.dpo_pair(cfg, 12, 4)
    loss, grads, _ = om.pref_step(cfg, P64, model, lora, c, c, 4, "simpo", beta=2.0, gamma=0.0)
    assert loss == pytest.approx(LN2, abs=1e-15)
    for l in range(cfg.L):
        for nm in om.NAMES:
            for w in range(2):
                assert np.abs(grads[l][nm][w]).max() < 1e-13
    _, g7, _ = om.pref_step(cfg, P64, model, lora, c, c, 4, "orpo", lam=0.7)
    _, g0, _ = om.pref_step(cfg, P64, model, lora, c, c, 4, "orpo", lam=0.0)
    for l in range(cfg.L):
        for nm in om.NAMES:
            for w in range(2):
                np.testing.assert_allclose(g7[l][nm][w], g0[l][nm][w], rtol=1e-9, atol=1e-13)


def test_kto_adapters_equal_reference():
    """LoRA B = 0: policy == reference, so both log ratios and z0 are 0 and the
    loss is (lam_d + lam_u) / 4 exactly; dA is zero."""
    cfg = MICRO
    model = oracle_model(cfg)
    c, r = synth.dpo_pair(cfg, 12, 4)
    loss, grads, aux = om.pref_step(cfg, PM, model, synth.lora_init(cfg, b_std=0.0), c, r, 4, "kto",
                                    beta=0.1, lam_d=1.0, lam_u=1.0)
    assert np.array_equal(aux["pi"], aux["ref"])
    assert loss == 0.5
    for l in range(cfg.L):
        for nm in om.NAMES:
            assert not np.any(grads[l][nm][0])
