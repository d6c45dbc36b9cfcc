"""GPU parity of the preference heads (DPO, SimPO, ORPO, KTO) on the tiny
stack, through the C ABI qls_pref_step, against oracle.model.pref_step:

  * loss within 1e-3 relative, LoRA gradients within 1e-2 relative L2 and
    cosine >= 0.999, response log-likelihood sums within 1e-3 relative;
  * KTO with LoRA B = 0 (policy == reference): loss exactly 1/2;
  * the reference-free heads stream the stack as an SFT step does (2L - 2
    layer loads) and give the same bits streamed and resident;
  * invalid configurations are refused before any launch.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from tests.gpu_util import bits, f32, report
from tests.test_gpu_step import _flat_oracle_grads, _setup

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")

PARAMS = {"dpo": {"beta": 0.1}, "simpo": {"beta": 2.0, "gamma": 0.5}, "orpo": {"lam": 0.25},
          "kto": {"beta": 0.3, "lam_d": 1.0, "lam_u": 1.3}}


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


@pytest.fixture(scope="module")
def tiny(q):
    cfg = synth.TINY
    store, model, res = _setup(q, cfg)
    return cfg, store, model, res


def _run(q, sess, cfg, kind, c, r, P, lora, **kw):
    d_lora = torch.from_numpy(synth.pack_lora(cfg, lora)).cuda()
    grads = torch.empty_like(d_lora)
    loss = torch.empty(1, device="cuda")
    aux = torch.empty(4, device="cuda")
    hl = sess.pref_step(kind, torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda(), P, d_lora, grads, loss,
                        aux, host_loss=True, **kw)
    torch.cuda.synchronize()
    return hl, grads, aux


@pytest.mark.parametrize("kind", ["dpo", "simpo", "orpo", "kto"])
def test_pref_matches_oracle(q, tiny, kind):
    cfg, store, model, res = tiny
    S, P = 64, 16
    c, r = synth.dpo_pair(cfg, S, P)
    lora = synth.lora_init(cfg, b_std=0.02)
    print(f"pref {kind} {PARAMS[kind]}", flush=True)
    sess = q.Session(store, *res, max_tokens=2 * S, max_seq=S)
    hl, grads, aux = _run(q, sess, cfg, kind, c, r, P, lora, **PARAMS[kind])
    ol, og, oaux = om.pref_step(cfg, PM, model, lora, c, r, P, kind, **PARAMS[kind])
    print(f"{kind} loss gpu={hl:.7f} oracle={ol:.7f} pi={oaux['pi']} ref={oaux['ref']}", flush=True)
    a = f32(aux)
    assert np.allclose(a[:2], oaux["pi"], rtol=1e-3)
    if kind in ("dpo", "kto"):
        assert np.allclose(a[2:], oaux["ref"], rtol=1e-3)
    else:
        assert not np.any(a[2:])
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    rr, cc = report(f"{kind} grads", grads.cpu().numpy(), _flat_oracle_grads(cfg, og))
    assert rr <= 1e-2 and cc >= 0.999
    sess.close()


def test_kto_b_zero_is_half(q, tiny):
    cfg, store, _, res = tiny
    c, r = synth.dpo_pair(cfg, 64, 16)
    sess = q.Session(store, *res, max_tokens=128, max_seq=64)
    hl, _, aux = _run(q, sess, cfg, "kto", c, r, 16, synth.lora_init(cfg, b_std=0.0), beta=0.1, lam_d=1.0,
                      lam_u=1.0)
    a = bits(aux)
    assert np.array_equal(a[:2], a[2:])
    assert hl == 0.5
    sess.close()


@pytest.mark.parametrize("kind", ["simpo", "orpo"])
def test_reference_free_streams_like_sft(q, tiny, kind):
    cfg, store, _, res = tiny
    c, r = synth.dpo_pair(cfg, 64, 16)
    lora = synth.lora_init(cfg, b_std=0.02)
    out = {}
    for mode in (q.QLS_STREAMED, q.QLS_RESIDENT):
        sess = q.Session(store, *res, max_tokens=128, max_seq=64, mode=mode)
        sess.reset_stats()
        hl, grads, aux = _run(q, sess, cfg, kind, c, r, 16, lora, **PARAMS[kind])
        if mode == q.QLS_STREAMED:
            assert sess.stats()["layer_loads"] == 2 * cfg.L - 2
        out[mode] = (np.float32(hl).view(np.uint32), bits(grads), bits(aux))
        sess.close()
    s, rr = out[q.QLS_STREAMED], out[q.QLS_RESIDENT]
    assert s[0] == rr[0] and np.array_equal(s[1], rr[1]) and np.array_equal(s[2], rr[2])


def test_invalid_configs_refused(q, tiny):
    cfg, store, _, res = tiny
    c, r = synth.dpo_pair(cfg, 64, 16)
    sess = q.Session(store, *res, max_tokens=128, max_seq=64)
    d_lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    grads = torch.empty_like(d_lora)
    loss = torch.empty(1, device="cuda")
    cc, rr = torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda()
    for kind, kw in [("dpo", {"beta": 0.0}), ("simpo", {"beta": -1.0}), ("kto", {"beta": float("nan")}),
                     ("orpo", {"lam": -0.1}), ("kto", {"beta": 0.1, "lam_u": -1.0})]:
        with pytest.raises(RuntimeError):
            sess.pref_step(kind, cc, rr, 16, d_lora, grads, loss, **kw)
    bad = q.PrefCfg(7, 0.1, 0.0, 0.0, 1.0, 1.0)
    with pytest.raises(RuntimeError):
        q.qls_pref_step(sess.h, bad, cc, rr, 64, 16, d_lora, grads, loss)
    sess.close()
