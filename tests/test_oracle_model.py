"""Pins for the oracle's decoder, hand-derived LoRA backward, CE and DPO (CPU only).

The pages print no worked loss or gradient, so the oracle is pinned to
mathematics and to independent library routines:
  * fp64 central finite differences of the loss (LoRA A/B entries, the
    embedded input, the DPO loss);
  * torch autograd through a forward built from torch library ops
    (F.rms_norm, scaled_dot_product_attention with GQA, complex-number RoPE,
    F.silu, F.cross_entropy) in float64;
  * identities: B = 0 gives the base output and dA = 0 exactly; the adapters-
    disabled reference pass equals the B = 0 policy; DPO with B = 0 gives
    loss ln 2 (page "Soup ... radar note", section "In detail": the DPO
    reference is the same base stream with the adapters disabled).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import model as om
from tests.helpers import MICRO, oracle_model, rel_l2

P64 = om.Prec("fp64")
PM = om.Prec("mirror")


def _loss64(cfg, model, lora, ids, x0=None):
    xs, _ = om.forward_sweep(cfg, P64, model, lora, ids, x0)
    hc = om.head_forward(cfg, P64, model, xs[-1])
    tgt = om.targets(ids)
    N = ids.shape[0] * (ids.shape[1] - 1)
    return float(-np.sum(om.row_logp(hc, tgt)) / N)


@pytest.fixture(scope="module")
def micro():
    cfg = MICRO
    model = oracle_model(cfg)
    lora = synth.lora_init(cfg, b_std=0.05)
    ids = synth.token_ids(cfg, 2, 12, seed=3)
    return cfg, model, lora, ids


def test_fd_lora_grads(micro):
    cfg, model, lora, ids = micro
    loss, grads, _ = om.sft_step(cfg, P64, model, lora, ids)
    assert abs(loss - _loss64(cfg, model, lora, ids)) < 1e-12
    rng = np.random.default_rng(0)
    h = 1e-5
    worst = 0.0
    for trial in range(70):
        l = int(rng.integers(cfg.L))
        name = om.NAMES[int(rng.integers(7))]
        which = int(rng.integers(2))
        M = lora[l][name][which]
        idx = tuple(int(rng.integers(s)) for s in M.shape)
        orig = float(M[idx])
        lp = [{n: (a.astype(np.float64).copy(), b.astype(np.float64).copy())
               for n, (a, b) in mods.items()} for mods in lora]
        Mp = lp[l][name][which]
        Mp[idx] = orig + h
        fp = _loss64(cfg, model, lp, ids)
        Mp[idx] = orig - h
        fm = _loss64(cfg, model, lp, ids)
        fd = (fp - fm) / (2 * h)
        an = grads[l][name][which][idx]
        # entries are 1e-4..1e-2; a dropped term or wrong sign is an O(1) error
        worst = max(worst, abs(fd - an) - 1e-5 * abs(an))
    assert worst < 1e-9, worst


def test_fd_input_grad(micro):
    cfg, model, lora, ids = micro
    x0 = P64.c(model.embed[ids.reshape(-1)])
    _, _, aux = om.sft_step(cfg, P64, model, lora, ids, x0=x0)
    g0 = aux["g0"]
    rng = np.random.default_rng(1)
    h = 1e-5
    for _ in range(25):
        idx = (int(rng.integers(x0.shape[0])), int(rng.integers(x0.shape[1])))
        xp = x0.copy(); xp[idx] += h
        xm = x0.copy(); xm[idx] -= h
        fd = (_loss64(cfg, model, lora, ids, xp) - _loss64(cfg, model, lora, ids, xm)) / (2 * h)
        assert abs(fd - g0[idx]) <= 1e-5 * abs(g0[idx]) + 1e-9, idx


def _torch_forward(cfg, model, lora_t, ids, B, S):
    """Float64 forward from torch library ops (independent of the oracle's code)."""
    dt = torch.float64
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=dt)
    s = cfg.alpha / cfg.r
    x = t(model.embed)[torch.as_tensor(ids.reshape(-1), dtype=torch.long)]
    inv = torch.tensor(float(cfg.theta), dtype=dt) ** (-torch.arange(0, cfg.hd, 2, dtype=dt) / cfg.hd)
    ang = torch.arange(S, dtype=dt)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)                        # e^{i angle}

    def rope(z, nh):                                                    # z [B*S, nh*hd]
        z = z.view(B, S, nh, cfg.hd)
        zc = torch.complex(z[..., :cfg.hd // 2], z[..., cfg.hd // 2:]) * rot[None, :, None, :]
        return torch.cat([zc.real, zc.imag], dim=-1)

    def lin(name, l, inp):
        A, Bm = lora_t[l][name]
        return inp @ t(model.layers[l]["W"][name]).T + s * (inp @ A.T) @ Bm.T

    for l in range(cfg.L):
        lw = model.layers[l]
        n1 = F.rms_norm(x, (cfg.d,), weight=t(lw["norm_attn"]), eps=cfg.eps)
        q = rope(lin("q", l, n1), cfg.H).transpose(1, 2)
        k = rope(lin("k", l, n1), cfg.KV).transpose(1, 2)
        v = lin("v", l, n1).view(B, S, cfg.KV, cfg.hd).transpose(1, 2)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
        o = o.transpose(1, 2).reshape(B * S, cfg.H * cfg.hd)
        hres = x + lin("o", l, o)
        n2 = F.rms_norm(hres, (cfg.d,), weight=t(lw["norm_mlp"]), eps=cfg.eps)
        x = hres + lin("down", l, F.silu(lin("gate", l, n2)) * lin("up", l, n2))
    hf = F.rms_norm(x, (cfg.d,), weight=t(model.final_norm), eps=cfg.eps)
    return hf @ t(model.lm_head).T


def test_autograd_fp64_matches_hand_backward(micro):
    cfg, model, lora, ids = micro
    B, S = ids.shape
    loss, grads, _ = om.sft_step(cfg, P64, model, lora, ids)
    lora_t = [{n: (torch.tensor(a, dtype=torch.float64, requires_grad=True),
                   torch.tensor(b, dtype=torch.float64, requires_grad=True))
               for n, (a, b) in mods.items()} for mods in lora]
    logits = _torch_forward(cfg, model, lora_t, ids, B, S).view(B, S, cfg.V)
    tl = F.cross_entropy(logits[:, :-1].reshape(-1, cfg.V),
                         torch.as_tensor(ids[:, 1:].reshape(-1), dtype=torch.long))
    tl.backward()
    assert abs(tl.item() - loss) < 1e-12 * max(1.0, abs(loss))
    for l in range(cfg.L):
        for n in om.NAMES:
            for w in range(2):
                ref = lora_t[l][n][w].grad.numpy()
                assert rel_l2(grads[l][n][w], ref) < 1e-9, (l, n, w)


def test_attention_matches_sdpa():
    rng = np.random.default_rng(2)
    B, S, H, KV, hd = 2, 9, 6, 2, 8
    q = rng.standard_normal((B * S, H, hd))
    k = rng.standard_normal((B * S, KV, hd))
    v = rng.standard_normal((B * S, KV, hd))
    o, lse = om.attention(P64, q, k, v, B, S)
    tq = torch.tensor(q).view(B, S, H, hd).transpose(1, 2)
    tk = torch.tensor(k).view(B, S, KV, hd).transpose(1, 2)
    tv = torch.tensor(v).view(B, S, KV, hd).transpose(1, 2)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    assert np.allclose(o, ref.transpose(1, 2).reshape(B * S, H, hd).numpy(), atol=1e-13)
    # KV == H reduces GQA to plain multi-head attention
    o2, _ = om.attention(P64, q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), B, S)
    assert np.allclose(o, o2, atol=1e-14)
    # lse against scipy-free direct form for one head
    s = (q[:S, 0] @ k[:S, 0].T) / math.sqrt(hd)
    s[np.triu_indices(S, 1)] = -np.inf
    assert np.allclose(lse[0, 0], np.log(np.exp(s).sum(1)), atol=1e-12)


def test_rope_properties():
    tabs = om.rope_tables(P64, 7, 16, 500000.0)
    x = np.random.default_rng(3).standard_normal((7, 3, 16))
    y = om.rope(P64, x, *tabs, 1)
    assert np.array_equal(y[0], x[0])                          # position 0: identity
    n_in = x[..., :8] ** 2 + x[..., 8:] ** 2
    n_out = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13)                # each pair keeps its norm
    back = om.rope(P64, y, *tabs, 1, inverse=True)
    assert np.allclose(back, x, atol=1e-13)
    # a single rotation by a known angle
    ang = 5 * 500000.0 ** (-2 * 3 / 16)
    assert np.isclose(y[5, 0, 3], x[5, 0, 3] * math.cos(ang) - x[5, 0, 11] * math.sin(ang))


def test_rmsnorm_constant_row():
    w = np.random.default_rng(4).standard_normal(32)
    for c in (0.5, -2.0, 7.0):
        y, _ = om.rmsnorm(P64, np.full((1, 32), c), w, 1e-5)
        assert np.allclose(y[0], c / math.sqrt(c * c + 1e-5) * w, rtol=1e-14)


def test_cross_entropy_matches_torch(micro):
    cfg, model, _, ids = micro
    xL = np.random.default_rng(5).standard_normal((ids.size, cfg.d))
    hc = om.head_forward(cfg, P64, model, xL)
    ours = -om.row_logp(hc, om.targets(ids)).reshape(ids.shape)[:, :-1]
    ref = F.cross_entropy(torch.tensor(hc["logits"]).view(*ids.shape, -1)[:, :-1].reshape(-1, cfg.V),
                          torch.as_tensor(ids[:, 1:].reshape(-1), dtype=torch.long), reduction="none")
    assert np.allclose(ours.reshape(-1), ref.numpy(), atol=1e-12)


def test_b_zero_gives_base_output_and_zero_dA():
    cfg = synth.TINY
    model = oracle_model(cfg)
    ids = synth.token_ids(cfg, 1, 64)
    lora0 = synth.lora_init(cfg, b_std=0.0)
    xs_pol, _ = om.forward_sweep(cfg, PM, model, lora0, ids)
    xs_ref, _ = om.forward_sweep(cfg, PM, model, None, ids)
    for a, b in zip(xs_pol, xs_ref):
        assert np.array_equal(a, b)
    _, grads, _ = om.sft_step(cfg, PM, model, lora0, ids)
    for l in range(cfg.L):
        for n in om.NAMES:
            assert not np.any(grads[l][n][0]), (l, n)          # dA == 0 exactly
            assert np.any(grads[l][n][1]), (l, n)              # dB carries signal


def test_reference_pass_equals_b_zero_policy():
    cfg = synth.TINY
    model = oracle_model(cfg)
    ids = synth.token_ids(cfg, 2, 32, seed=9)
    ref, lp_ref = om.seq_logprobs(cfg, PM, model, None, ids, 8)
    pol, lp_pol = om.seq_logprobs(cfg, PM, model, synth.lora_init(cfg, b_std=0.0), ids, 8)
    assert np.array_equal(lp_ref, lp_pol) and np.array_equal(ref, pol)
    pol2, _ = om.seq_logprobs(cfg, PM, model, synth.lora_init(cfg, b_std=0.01), ids, 8)
    assert not np.array_equal(ref, pol2)


@pytest.mark.parametrize("P", [P64, PM], ids=["fp64", "mirror"])
def test_dpo_b_zero_is_ln2(P):
    cfg = MICRO
    model = oracle_model(cfg)
    c, r = synth.dpo_pair(cfg, 12, 4)
    beta = 0.1
    loss, grads, aux = om.dpo_step(cfg, P, model, synth.lora_init(cfg, b_std=0.0), c, r, 4, beta)
    assert aux["z"] == 0.0
    assert loss == math.log(2.0)
    for l in range(cfg.L):
        for n in om.NAMES:
            assert not np.any(grads[l][n][0])


def test_dpo_fd():
    cfg = MICRO
    model = oracle_model(cfg)
    lora = synth.lora_init(cfg, b_std=0.05)
    c, r = synth.dpo_pair(cfg, 12, 4)
    beta = 0.1
    loss, grads, _ = om.dpo_step(cfg, P64, model, lora, c, r, 4, beta)
    rng = np.random.default_rng(6)
    h = 1e-5
    for _ in range(20):
        l = int(rng.integers(cfg.L)); n = om.NAMES[int(rng.integers(7))]; w = int(rng.integers(2))
        M = lora[l][n][w]
        idx = tuple(int(rng.integers(s)) for s in M.shape)
        vals = []
        for sgn in (1, -1):
            lp = [{k: (a.astype(np.float64).copy(), b.astype(np.float64).copy())
                   for k, (a, b) in mods.items()} for mods in lora]
            lp[l][n][w][idx] += sgn * h
            vals.append(om.dpo_step(cfg, P64, model, lp, c, r, 4, beta)[0])
        fd = (vals[0] - vals[1]) / (2 * h)
        an = grads[l][n][w][idx]
        assert abs(fd - an) <= 1e-5 * abs(an) + 1e-10, (l, n, w, fd, an)


def test_sft_loss_near_ln_vocab():
    """Random init: logits are nearly uniform, so the loss sits near ln V
    (approximate sanity check, not a pin)."""
    cfg = synth.TINY
    model = oracle_model(cfg, perturbed=False)
    ids = synth.token_ids(cfg, 1, 64)
    loss, _, _ = om.sft_step(cfg, PM, model, synth.lora_init(cfg), ids)
    assert abs(loss - math.log(cfg.V)) < 0.5


def test_response_logprob_span_matches_torch_cross_entropy(micro):
    """The response log-likelihood of a (prompt, response) sequence is the sum,
    over every response token at position t in [P, S), of log p(ids_t |
    ids_<t), the next-token distribution read from the logits of position t-1.
    Written here position by position with torch's F.cross_entropy on logits
    from the library-op forward, independent of the oracle's row / span
    bookkeeping; seq_logprobs, dpo_step and pref_step must all agree."""
    cfg, model, lora, _ = micro
    S, P, beta = 12, 4, 0.1
    c, r = synth.dpo_pair(cfg, S, P, seeds=(61, 62, 63))
    ids2 = np.stack([c, r])
    tid = torch.as_tensor(ids2, dtype=torch.long)

    def torch_pi(lr, lo=P, hi=S):
        lt = [{n: (torch.tensor(a, dtype=torch.float64), torch.tensor(b, dtype=torch.float64))
               for n, (a, b) in mods.items()} for mods in lr]
        with torch.no_grad():
            logits = _torch_forward(cfg, model, lt, ids2, 2, S).view(2, S, cfg.V)
        return [sum(-F.cross_entropy(logits[b, t - 1][None], tid[b, t][None]).item() for t in range(lo, hi))
                for b in range(2)]

    pol = torch_pi(lora)
    ref = torch_pi(synth.lora_init(cfg, b_std=0.0))          # adapters disabled: B = 0
    pol_shift = torch_pi(lora, lo=P - 1, hi=S - 1)           # the span one position early
    seq, _ = om.seq_logprobs(cfg, P64, model, lora, ids2, P)
    seq_ref, _ = om.seq_logprobs(cfg, P64, model, None, ids2, P)
    assert np.allclose(seq, pol, rtol=1e-11, atol=0) and np.allclose(seq_ref, ref, rtol=1e-11, atol=0)
    loss, _, aux = om.dpo_step(cfg, P64, model, lora, c, r, P, beta)
    assert np.allclose(aux["pi"], pol, rtol=1e-11) and np.allclose(aux["ref"], ref, rtol=1e-11)
    z = beta * ((pol[0] - ref[0]) - (pol[1] - ref[1]))
    assert abs(loss - math.log1p(math.exp(-z))) < 1e-12
    _, _, paux = om.pref_step(cfg, P64, model, lora, c, r, P, "simpo", beta=2.0, gamma=1.0)
    assert np.allclose(paux["pi"], pol, rtol=1e-11)
    # an off-by-one span would be seen: the sums one position early differ
    assert np.all(np.abs(np.asarray(pol_shift) - seq) > 1e-3)
