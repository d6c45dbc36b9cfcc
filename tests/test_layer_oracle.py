"""The per-layer oracle workers (tests/layer_oracle.py) reproduce the oracle's
own layer-by-layer backward sweep: fed the oracle's checkpoints x_l and the
gradients dL/dx_{l+1} of an oracle SFT step, every layer's output, dL/dx_l
and LoRA gradients equal those of the step bit for bit.  This pins the
plumbing of the per-layer check (layer indices, boundary entries, LoRA
slices, seeded weights) that the 8B GPU tests rely on."""
import numpy as np

import synth
from oracle import model as om
from tests.helpers import oracle_model
from tests.layer_oracle import run_layers


def test_workers_reproduce_the_oracle_sweep():
    cfg = synth.TINY
    P = om.Prec("mirror")
    model = oracle_model(cfg, perturbed=False)
    lora = synth.lora_init(cfg)
    ids = synth.token_ids(cfg, 1, 64)
    loss, grads, aux = om.sft_step(cfg, P, model, lora, ids)
    xs = aux["xs"]
    # the gradient at every layer boundary, by the oracle's own sweep
    B, S = ids.shape
    tabs = om.rope_tables(P, S, cfg.hd, cfg.theta)
    hc = om.head_forward(cfg, P, model, xs[-1])
    tgt = om.targets(ids)
    w = np.where(tgt >= 0, 1.0 / (B * (S - 1)), 0.0)
    g = [None] * (cfg.L + 1)
    g[cfg.L] = om.head_backward(cfg, P, model, xs[-1], hc, tgt, w)
    for l in reversed(range(cfg.L)):
        _, c = om.layer_forward(cfg, P, xs[l], model.layers[l], lora[l], B, S, tabs)
        g[l], _ = om.layer_backward(cfg, P, c, g[l + 1], model.layers[l], lora[l], B, S, tabs)
    assert np.array_equal(g[0], aux["g0"])
    jobs = [(cfg, l, xs[l], np.asarray(g[l + 1], np.float32), lora[l], B, S, "f32", False)
            for l in range(cfg.L)]
    res = run_layers(jobs, workers=2, threads=2)
    for l in range(cfg.L):
        out, g_in, og = res[l]
        assert np.array_equal(out, xs[l + 1]), l
        assert np.array_equal(g_in, np.asarray(g[l], np.float32)), l
        for n in om.NAMES:
            for k in range(2):
                assert np.array_equal(og[n][k], grads[l][n][k]), (l, n, k)
