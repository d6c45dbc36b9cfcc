"""Pins for the oracle's AdamW (CPU only): torch.optim.AdamW, an independent
library implementation, in float64 over several steps; mirror precision within
float32 rounding of it."""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import optim


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_adamw_matches_torch_float64(wd):
    rng = np.random.default_rng(0)
    n, steps, lr = 4096, 6, 2e-3
    p0 = rng.normal(0, 0.05, n)
    grads = [rng.normal(0, 1e-2, n) * (1 + i) for i in range(steps)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd)
    P = om.Prec("fp64")
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = optim.adamw_step(P, p, g, m, v, t, lr, wd=wd)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-11, atol=1e-16)
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-11)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-11)


def test_adamw_mirror_close_to_fp64_and_first_step_closed_form():
    rng = np.random.default_rng(1)
    n, lr = 10000, 2e-5
    p0 = rng.normal(0, 0.05, n).astype(np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    z = np.zeros(n, np.float32)
    p32, _, _ = optim.adamw_step(om.Prec("mirror"), p0, g, z, z, 1, lr)
    p64, _, _ = optim.adamw_step(om.Prec("fp64"), p0, g, z, z, 1, lr)
    assert p32.dtype == np.float32
    np.testing.assert_allclose(p32, p64, rtol=2e-7, atol=1e-9)
    # step 1 from m = v = 0: the bias corrections cancel, so p1 = p0 - lr g / (|g| + eps)
    g64 = g.astype(np.float64)
    want = p0.astype(np.float64) - lr * g64 / (np.abs(g64) + 1e-8)
    np.testing.assert_allclose(p64, want, rtol=1e-12, atol=1e-15)
