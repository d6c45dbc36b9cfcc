"""GPU parity at the 8B shape, through the C ABI.

* One Llama-3.1-8B-shaped decoder layer streamed from pinned host memory,
  forward + recomputed forward + backward, against the oracle run on the same
  seeded inputs (rel. L2 <= 1e-2, cosine >= 0.999 for the output, dL/dx and
  every LoRA matrix), and streamed == resident bitwise; the same for a
  narrower layer at 8192 tokens, which takes the large-tile GEMM kernels.
* A layer above 172 MiB (hidden 5120, SwiGLU 27648: 274 MB per record) streams
  bit-identically to the resident run -- page "Can You Fine-Tune Llama 3.1 8B
  on a 4GB GPU? ...", section "Did a correctness bug invalidate the Llama 3.1
  8B result?": wrong gradients appeared between 163.8 and 171.5 MiB per layer.
* The full 32-layer step at seq 512: streamed == resident bitwise (loss, every
  checkpoint, every gradient) and loss / gradients against the oracle's golden
  values in mirror and in fp64 precision (tests/golden/sft_8b_seq512.json and
  sft_8b_seq512_fp64.json, written by make_golden_8b.py).
* DPO on the full stack: the fused reference equals the adapters-disabled
  log-prob pass bit for bit, and B = 0 gives loss ln 2.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from tests.gpu_util import bits, f32, report
from tests.helpers import cosine, rel_l2

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sft_8b_seq512.json")
GOLDEN64 = os.path.join(os.path.dirname(__file__), "golden", "sft_8b_seq512_fp64.json")


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _store(q, cfg, threads=8):
    store = q.Store(cfg)
    for l in range(cfg.L):
        na, nm = synth.layer_norms(cfg, l)
        store.set_layer_fp32(l, synth.base_layer(cfg, l, threads=threads), na, nm, n_threads=threads)
    return store


def _grad_check(name, got, want):
    r, c = report(name, got, want)
    assert r <= 1e-2 and c >= 0.999, (name, r, c)


# (config, batch, seq): one 8B layer at 512 tokens, and a narrower layer at
# 4 x 2048 tokens whose every projection (fused q|k|v with three LoRA modules,
# o and down with the residual, gate|up) and every dX product is large enough
# for the 256 x 256 dequant-GEMM kernels.
WIDE = synth.ModelCfg(L=1, d=2048, H=16, KV=4, hd=128, I=5632, V=1024, eps=1e-5, theta=500000.0,
                      r=16, alpha=32.0)
LAYER_CASES = [("8b", synth.scaled(synth.LLAMA8B, L=1), 1, 512), ("wide-8k-tokens", WIDE, 4, 2048)]


@pytest.mark.parametrize("name,cfg,B,S", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_one_layer_matches_oracle(q, name, cfg, B, S):
    T = B * S
    print(f"building one layer ({name}, {B} x {S} tokens)", flush=True)
    store = _store(q, cfg)
    emb = torch.zeros(cfg.V, cfg.d, dtype=torch.bfloat16, device="cuda")   # unused by a single layer
    fn = torch.ones(cfg.d, dtype=torch.bfloat16, device="cuda")
    lora = synth.lora_init(cfg, b_std=1e-2)
    d_lora = torch.from_numpy(synth.pack_lora(cfg, lora)).cuda()
    x = synth.activation(31, (T, cfg.d))
    gout = synth.activation(32, (T, cfg.d))
    res = {}
    for mode in (q.QLS_STREAMED, q.QLS_RESIDENT):
        sess = q.Session(store, emb, emb, fn, max_tokens=T, max_seq=S, mode=mode)
        out = torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda")
        gin = torch.empty(T, cfg.d, dtype=torch.float32, device="cuda")
        grads = torch.zeros_like(d_lora)
        sess.layer_fwd_bwd(0, x.cuda(), gout.cuda(), B, S, d_lora, out, gin, grads)
        torch.cuda.synchronize()
        res[mode] = (out.cpu(), gin.cpu(), grads.cpu())
        sess.close()
    for a, b in zip(res[q.QLS_STREAMED], res[q.QLS_RESIDENT]):
        assert np.array_equal(bits(a), bits(b))
    print("oracle: quantising and running the layer", flush=True)
    ws = synth.base_layer(cfg, 0, threads=8)
    na, nm = synth.layer_norms(cfg, 0)
    lw = om.dequant_layer(cfg, ws, na.float().numpy(), nm.float().numpy())
    del ws
    tabs = om.rope_tables(PM, S, cfg.hd, cfg.theta)
    xo = x.float().numpy()
    out_o, cache = om.layer_forward(cfg, PM, xo, lw, lora[0], B, S, tabs)
    gin_o, grads_o = om.layer_backward(cfg, PM, cache, gout.float().numpy(), lw, lora[0], B, S, tabs)
    out, gin, grads = res[q.QLS_STREAMED]
    _grad_check("layer out", f32(out), out_o)
    _grad_check("dL/dx", f32(gin), gin_o)
    per = synth.unpack_lora(cfg, grads.numpy())
    for n in om.NAMES:
        for w in range(2):
            _grad_check(f"{n}.{'AB'[w]}", per[0][n][w], grads_o[n][w])


def test_layer_above_172_mib_streams_bit_identically(q):
    cfg = synth.ModelCfg(L=3, d=5120, H=40, KV=8, hd=128, I=27648, V=1024, eps=1e-5, theta=500000.0,
                         r=16, alpha=32.0)
    rec = q.qls_layer_record_bytes(q.model_cfg(cfg))
    assert rec > 172 * 2 ** 20, rec
    print(f"record {rec / 2 ** 20:.1f} MiB", flush=True)
    store = _store(q, cfg)
    emb, lm, fn = synth.embedding(cfg).cuda(), synth.lm_head(cfg).cuda(), synth.final_norm(cfg).cuda()
    ids = torch.from_numpy(synth.token_ids(cfg, 1, 64, seed=5)).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=1e-2))).cuda()
    out = {}
    for name, mode, flags in [("resident", q.QLS_RESIDENT, 0), ("streamed", q.QLS_STREAMED, 0),
                              ("poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE)]:
        sess = q.Session(store, emb, lm, fn, max_tokens=64, max_seq=64, mode=mode)
        sess.debug(flags)
        grads = torch.full_like(lora, float("nan"))
        loss = torch.empty(1, device="cuda")
        sess.sft_step(ids, lora, grads, loss)
        torch.cuda.synchronize()
        out[name] = (bits(loss), bits(grads), bits(sess.checkpoints(64)))
        sess.close()
    for name in ("streamed", "poison"):
        for a, b in zip(out[name], out["resident"]):
            assert np.array_equal(a, b), name
    assert np.all(np.isfinite(out["resident"][1].view(np.float32)))


@pytest.fixture(scope="module")
def stack8b(q):
    cfg = synth.LLAMA8B
    print("building the 32-layer 8B store", flush=True)
    store = _store(q, cfg, threads=16)
    res = (synth.embedding(cfg, threads=16).cuda(), synth.lm_head(cfg, threads=16).cuda(),
           synth.final_norm(cfg).cuda())
    return cfg, store, res


def test_full_8b_step_streamed_equals_resident_and_oracle(q, stack8b):
    cfg, store, res = stack8b
    S = 512
    ids = torch.from_numpy(synth.token_ids(cfg, 1, S, seed=41)).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    runs = {}
    for mode in (q.QLS_STREAMED, q.QLS_RESIDENT):
        print(f"8B step mode {mode}", flush=True)
        sess = q.Session(store, *res, max_tokens=S, max_seq=S, mode=mode)
        grads = torch.full_like(lora, float("nan"))
        loss = torch.empty(1, device="cuda")
        hl = sess.sft_step(ids, lora, grads, loss, host_loss=True)
        runs[mode] = (hl, bits(loss), bits(sess.checkpoints(S)), grads.cpu())
        sess.close()
    s, r = runs[q.QLS_STREAMED], runs[q.QLS_RESIDENT]
    assert np.array_equal(s[1], r[1])                      # loss
    assert np.array_equal(s[2], r[2])                      # forward question: every checkpoint
    assert np.array_equal(bits(s[3]), bits(r[3]))          # gradient question: every dA / dB
    hl, grads = s[0], s[3].numpy()
    assert np.all(np.isfinite(grads))
    print(f"8B loss {hl:.6f} (ln V = {math.log(cfg.V):.4f})", flush=True)
    if not (os.path.exists(GOLDEN) and os.path.exists(GOLDEN64)):
        pytest.skip("golden values not generated (tests/golden/make_golden_8b.py)")
    mir, ref = json.load(open(GOLDEN)), json.load(open(GOLDEN64))
    # Loss: within 1e-3 of both the mirror-precision oracle and the fp64 oracle.
    for gold in (mir, ref):
        assert abs(hl - gold["loss"]) <= 1e-3 * abs(gold["loss"]), (hl, gold["loss"])
    per = synth.unpack_lora(cfg, grads)
    got = np.array([per[l][om.NAMES[m]][w].reshape(-1)[i] for l, m, w, i, _ in mir["samples"]])
    want_m = np.array([v for *_, v in mir["samples"]])
    want_f = np.array([v for *_, v in ref["samples"]])
    gn = np.array([np.linalg.norm(per[l][om.NAMES[m]][w].astype(np.float64)) for l, m, w, _ in mir["grad_norms"]])
    wn_m = np.array([v for *_, v in mir["grad_norms"]])
    wn_f = np.array([v for *_, v in ref["grad_norms"]])
    # Through 32 bf16 layers, rounding-order differences compound: the mirror
    # oracle itself sits ~9% (rel. L2, cos ~0.996) from the fp64 oracle on these
    # entries, so the per-entry 1e-2 bar (met per layer above) cannot hold for
    # the whole stack.  The GPU must be as close to fp64 as the mirror oracle is
    # (25% slack), and near the mirror oracle itself.
    r_gpu, c_gpu = report("sampled grads vs fp64 oracle", got, want_f)
    r_mir, c_mir = report("mirror oracle vs fp64 oracle", want_m, want_f)
    assert r_gpu <= 1.25 * r_mir and c_gpu >= c_mir - 1e-3, (r_gpu, r_mir, c_gpu, c_mir)
    r_gm, c_gm = report("sampled grads vs mirror oracle", got, want_m)
    assert r_gm <= 0.1 and c_gm >= 0.995, (r_gm, c_gm)
    # Per-matrix gradient norms: as close to fp64 as the mirror oracle's (25%
    # slack), and within 1e-2 of the mirror oracle.
    e_gpu = np.max(np.abs(gn - wn_f) / wn_f)
    e_mir = np.max(np.abs(wn_m - wn_f) / wn_f)
    print(f"grad norms: max rel vs fp64 {e_gpu:.3e} (mirror {e_mir:.3e}), vs mirror "
          f"{np.max(np.abs(gn - wn_m) / wn_m):.3e}", flush=True)
    assert e_gpu <= 1.25 * e_mir, (e_gpu, e_mir)
    assert np.max(np.abs(gn - wn_m) / wn_m) <= 1e-2


def test_full_8b_dpo_reference_and_b_zero(q, stack8b):
    cfg, store, res = stack8b
    S, P, beta = 512, 128, 0.1
    c, r = synth.dpo_pair(cfg, S, P)
    ids2 = torch.from_numpy(np.stack([c, r])).cuda()
    sess = q.Session(store, *res, max_tokens=2 * S, max_seq=S)
    ref = torch.empty(2, device="cuda")
    sess.logprobs(ids2, P, None, ref)
    for b_std in (1e-3, 0.0):
        lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=b_std))).cuda()
        grads = torch.full_like(lora, float("nan"))
        loss = torch.empty(1, device="cuda")
        aux = torch.empty(4, device="cuda")
        hl = sess.dpo_step(ids2[0].contiguous(), ids2[1].contiguous(), P, beta, lora, grads, loss, aux,
                           host_loss=True)
        a = bits(aux)
        assert np.array_equal(a[2:], bits(ref))           # fused reference == standalone pass
        assert bool(torch.isfinite(grads).all())
        if b_std == 0.0:
            assert np.array_equal(a[:2], a[2:]) and hl == np.float32(math.log(2.0))
        print(f"dpo b_std={b_std}: loss {hl:.6f}, logp {f32(aux)}", flush=True)
    sess.close()
