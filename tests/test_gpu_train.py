"""The training loop around the streamed step: AdamW on the LoRA vector.

* The device AdamW equals the oracle's (mirror precision) bit for bit.
* 20 streamed steps against 20 resident steps (page "Fine-Tune an 8B Model on
  a 4GB Laptop GPU: Hands-On Guide", section "The gotchas nobody's mentioning
  yet": matching loss curves as the practical check): the loss curves, the
  final LoRA vector and the optimizer moments are identical bit for bit, also
  with slots poisoned on release and with AdamW folded into the backward
  sweep (qls_sft_step_adamw).
* The same 20-step loop against the oracle's: every step's loss within 1e-3
  relative; the LoRA change over the 20 steps within 3e-2 relative L2 and
  cosine 0.999.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from oracle import optim
from tests.gpu_util import bits, report

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def test_adamw_bitwise_equals_oracle(q):
    rng = np.random.default_rng(5)
    n = 100_003
    p = rng.normal(0, 0.05, n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dp, dm, dv = (torch.from_numpy(x.copy()).cuda() for x in (p, m, v))
    for t in range(1, 5):
        g = (rng.normal(0, 1e-3, n) * t).astype(np.float32)
        q.qls_adamw_step(dp, torch.from_numpy(g).cuda(), dm, dv, t, 1e-3, weight_decay=0.01)
        p, m, v = optim.adamw_step(PM, p, g, m, v, t, 1e-3, wd=0.01)
    torch.cuda.synchronize()
    for got, want in ((dp, p), (dm, m), (dv, v)):
        assert np.array_equal(bits(got), want.view(np.uint32))


def _loop(q, store, res, cfg, ids, steps, lr, mode, flags=0, fused=False):
    sess = q.Session(store, *res, max_tokens=ids.shape[0] * ids.shape[1], max_seq=ids.shape[1], mode=mode)
    sess.debug(flags)
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=0.0))).cuda()
    opt = q.AdamW(lora, lr=lr)
    grads = torch.empty_like(lora)
    loss = torch.empty(1, device="cuda")
    d_ids = torch.from_numpy(ids).cuda()
    curve = []
    for _ in range(steps):
        if fused:
            curve.append(sess.sft_step_adamw(d_ids, opt, grads, loss, host_loss=True))
            continue
        curve.append(sess.sft_step(d_ids, lora, grads, loss, host_loss=True))
        opt.step(grads)
    torch.cuda.synchronize()
    sess.close()
    return np.array(curve, np.float32), lora, opt


def _store(q, cfg):
    store = q.Store(cfg)
    layers = []
    for l in range(cfg.L):
        ws = synth.base_layer(cfg, l)
        na, nm = synth.layer_norms(cfg, l, True)
        store.set_layer_fp32(l, ws, na, nm)
        layers.append(om.dequant_layer(cfg, ws, na.float().numpy(), nm.float().numpy()))
    emb, lm, fn = synth.embedding(cfg), synth.lm_head(cfg), synth.final_norm(cfg, True)
    model = om.Model(cfg, layers, emb.float().numpy(), lm.float().numpy(), fn.float().numpy())
    return store, model, (emb.cuda(), lm.cuda(), fn.cuda())


def test_20_streamed_steps_equal_20_resident_steps(q):
    cfg = synth.scaled(synth.TINY, L=6)
    store, _, res = _store(q, cfg)
    ids = synth.token_ids(cfg, 1, 64, seed=11)
    runs = {name: _loop(q, store, res, cfg, ids, 20, 1e-3, mode, flags, fused)
            for name, mode, flags, fused in [("resident", q.QLS_RESIDENT, 0, False),
                                             ("streamed", q.QLS_STREAMED, 0, False),
                                             ("poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE, False),
                                             ("fused", q.QLS_STREAMED, 0, True),
                                             ("fused-poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE, True)]}
    curve = runs["resident"][0]
    print("loss curve", np.round(curve, 5).tolist(), flush=True)
    assert curve[-1] < curve[0]                               # it trains
    for name in ("streamed", "poison", "fused", "fused-poison"):
        c, p, o = runs[name]
        assert np.array_equal(c.view(np.uint32), curve.view(np.uint32)), name
        assert np.array_equal(bits(p), bits(runs["resident"][1])), name
        assert np.array_equal(bits(o.m), bits(runs["resident"][2].m)), name
        assert np.array_equal(bits(o.v), bits(runs["resident"][2].v)), name


def test_20_step_loop_matches_oracle_loop(q):
    cfg = synth.TINY
    store, model, res = _store(q, cfg)
    ids = synth.token_ids(cfg, 1, 64, seed=12)
    steps, lr = 20, 1e-3
    curve, lora_gpu, _ = _loop(q, store, res, cfg, ids, steps, lr, q.QLS_STREAMED)
    lora = synth.lora_init(cfg, b_std=0.0)
    p = synth.pack_lora(cfg, lora)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    want = []
    for t in range(1, steps + 1):
        loss, grads, _ = om.sft_step(cfg, PM, model, synth.unpack_lora(cfg, p), ids)
        want.append(loss)
        g = np.concatenate([np.concatenate([grads[l][n][0].ravel(), grads[l][n][1].ravel()])
                            for l in range(cfg.L) for n in om.NAMES]).astype(np.float32)
        p, m, v = optim.adamw_step(PM, p, g, m, v, t, lr)
    want = np.array(want)
    print("gpu", np.round(curve, 5).tolist(), "\\noracle", np.round(want, 5).tolist(), flush=True)
    assert np.all(np.abs(curve - want) <= 1e-3 * np.abs(want)), np.max(np.abs(curve - want) / np.abs(want))
    # AdamW moves every entry by about lr * sign(m), whatever the gradient's
    # size, so entries whose gradients are rounding noise move differently in
    # the two runs: the parameter change gets 3e-2 (per-step losses are the
    # primary check above).
    r, c = report("LoRA change after 20 steps", lora_gpu.cpu().numpy() - synth.pack_lora(cfg, lora),
                  p - synth.pack_lora(cfg, lora))
    assert r <= 3e-2 and c >= 0.999
