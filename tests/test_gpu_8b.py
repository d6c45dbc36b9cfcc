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
  checkpoint, every gradient); every layer of the real step checked against
  the oracle at the gradient bar (rel. L2 <= 1e-2, cosine >= 0.999 for each
  of its 14 LoRA matrices, its output and dL/dx), the oracle given the
  layer's input checkpoint and the float32 gradient arriving from above
  (page "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU? ...", section "The
  gradient bug also reveals something important about AI benchmarks": the
  gradients are checked on their own); the loss against the oracle's golden
  value in mirror and in fp64 precision, and the whole-stack gradients against
  both as a propagation check (tests/golden/sft_8b_seq512*.json, written by
  make_golden_8b.py).
* The full step at seq 4096: streamed == resident bitwise, layers 0 and 31
  against the oracle at the gradient bar, the loss against the golden value
  (tests/golden/sft_8b_seq4096.json).
* DPO on the full stack (chosen and rejected 1 x 512 sharing a 128-token
  prompt): streamed == resident bitwise (loss, pi / rho, every gradient), the
  fused reference equals the adapters-disabled log-prob pass bit for bit,
  layers 0, 16 and 31 against the oracle at the gradient bar, pi and rho within
  1e-3 of the mirror and fp64 oracles' golden values, the loss, z and the
  whole-stack gradients as close to the fp64 oracle as the mirror oracle is
  (tests/golden/dpo_8b_seq512*.json), and B = 0 gives loss ln 2.
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
from tests.layer_oracle import cpu_share, run_layers

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sft_8b_seq512.json")
GOLDEN64 = os.path.join(os.path.dirname(__file__), "golden", "sft_8b_seq512_fp64.json")
GOLDEN4096 = os.path.join(os.path.dirname(__file__), "golden", "sft_8b_seq4096.json")
GOLDEN_DPO = os.path.join(os.path.dirname(__file__), "golden", "dpo_8b_seq512.json")
GOLDEN_DPO64 = os.path.join(os.path.dirname(__file__), "golden", "dpo_8b_seq512_fp64.json")


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


def _sft_run(q, cfg, store, res, ids, lora, mode, capture):
    """One SFT step; returns host copies of the loss (float and bits), every
    checkpoint (bf16 bits), the gradients and, with capture, the float32
    residual gradient at every layer boundary ([L+1, T, d])."""
    B, S = ids.shape
    T = B * S
    sess = q.Session(store, *res, max_tokens=T, max_seq=S, mode=mode)
    cap = None
    if capture:
        cap = torch.full(((cfg.L + 1) * T * cfg.d,), float("nan"), device="cuda")
        sess.capture_grads(cap)
    grads = torch.full_like(lora, float("nan"))
    loss = torch.empty(1, device="cuda")
    hl = sess.sft_step(ids, lora, grads, loss, host_loss=True)
    out = {"hl": hl, "loss": bits(loss), "ck": bits(sess.checkpoints(T)), "grads": grads.cpu()}
    if capture:
        out["cap"] = cap.view(cfg.L + 1, T, cfg.d).cpu().numpy()
    sess.close()
    return out


def _per_layer_check(cfg, layers, ck_bits, cap, grads, lora, B, S, workers, threads):
    """Each listed layer of a real step through the oracle, given that layer's
    input checkpoint and the float32 gradient arriving from above: its output
    (the next checkpoint), dL/dx and its 14 LoRA gradient matrices must each be
    within rel. L2 1e-2 and cosine 0.999 of the oracle's."""
    ck = (ck_bits.astype(np.uint32) << 16).view(np.float32)
    jobs = [(cfg, l, ck[l], cap[l + 1], lora[l], B, S, "f32", False) for l in layers]
    res = run_layers(jobs, workers, threads)
    per = synth.unpack_lora(cfg, grads.numpy() if hasattr(grads, "numpy") else grads)
    worst = (0.0, 1.0, "")
    fails = []
    for l in layers:
        out, g_in, og = res[l]
        pairs = [("out", ck[l + 1], out), ("dL/dx", cap[l], g_in)]
        pairs += [(f"{n}.{'AB'[w]}", per[l][n][w], og[n][w]) for n in om.NAMES for w in range(2)]
        lw = (0.0, 1.0)
        for name, got, want in pairs:
            r, c = rel_l2(got, want), cosine(got, want)
            lw = (max(lw[0], r), min(lw[1], c))
            if r > worst[0]:
                worst = (r, min(worst[1], c), f"layer {l} {name}")
            if not (r <= 1e-2 and c >= 0.999):
                fails.append((l, name, r, c))
        print(f"layer {l}: worst rel_l2 {lw[0]:.3e}, worst cos {lw[1]:.7f} over out, dL/dx and 14 LoRA "
              f"gradients", flush=True)
    print(f"per-layer check over layers {list(layers)}: worst rel_l2 {worst[0]:.3e} ({worst[2]})", flush=True)
    assert not fails, fails


@pytest.fixture(scope="module")
def sft512(q, stack8b):
    cfg, store, res = stack8b
    S = 512
    ids = torch.from_numpy(synth.token_ids(cfg, 1, S, seed=41)).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    print("8B step, streamed (gradients captured at every layer boundary)", flush=True)
    s = _sft_run(q, cfg, store, res, ids, lora, q.QLS_STREAMED, capture=True)
    print("8B step, resident", flush=True)
    r = _sft_run(q, cfg, store, res, ids, lora, q.QLS_RESIDENT, capture=False)
    return s, r


def test_full_8b_step_streamed_equals_resident(q, stack8b, sft512):
    cfg = stack8b[0]
    s, r = sft512
    assert np.array_equal(s["loss"], r["loss"])                     # loss
    assert np.array_equal(s["ck"], r["ck"])                         # forward question: every checkpoint
    assert np.array_equal(bits(s["grads"]), bits(r["grads"]))       # gradient question: every dA / dB
    assert np.all(np.isfinite(s["grads"].numpy()))
    assert np.all(np.isfinite(s["cap"]))
    print(f"8B loss {s['hl']:.6f} (ln V = {math.log(cfg.V):.4f})", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("group", range(4))
def test_full_8b_step_every_layer_matches_oracle(stack8b, sft512, group):
    """Layers 8*group .. 8*group+7 of the seq-512 step, eight at a time."""
    cfg = stack8b[0]
    s, _ = sft512
    n = cpu_share()
    workers = max(1, min(8, n // 2))
    layers = range(8 * group, 8 * group + 8)
    _per_layer_check(cfg, layers, s["ck"], s["cap"], s["grads"], synth.lora_init(cfg), 1, 512, workers,
                     max(1, n // workers))


def test_full_8b_step_loss_and_propagation(stack8b, sft512):
    """Loss within 1e-3 of the oracle in mirror and fp64 precision.  The
    whole-stack gradients are a propagation check, not the gradient bar (that
    bar holds layer by layer above): through 32 bf16 layers the mirror oracle
    itself sits ~9% (rel. L2) from the fp64 oracle on the sampled entries, so
    rounding-order differences compound; the GPU must be as close to fp64 as
    the mirror oracle is (25% slack)."""
    cfg = stack8b[0]
    s, _ = sft512
    if not (os.path.exists(GOLDEN) and os.path.exists(GOLDEN64)):
        pytest.skip("golden values not generated (tests/golden/make_golden_8b.py)")
    hl, grads = s["hl"], s["grads"].numpy()
    mir, ref = json.load(open(GOLDEN)), json.load(open(GOLDEN64))
    for gold in (mir, ref):
        assert abs(hl - gold["loss"]) <= 1e-3 * abs(gold["loss"]), (hl, gold["loss"])
    per = synth.unpack_lora(cfg, grads)
    got = np.array([per[l][om.NAMES[m]][w].reshape(-1)[i] for l, m, w, i, _ in mir["samples"]])
    want_m = np.array([v for *_, v in mir["samples"]])
    want_f = np.array([v for *_, v in ref["samples"]])
    gn = np.array([np.linalg.norm(per[l][om.NAMES[m]][w].astype(np.float64)) for l, m, w, _ in mir["grad_norms"]])
    wn_m = np.array([v for *_, v in mir["grad_norms"]])
    wn_f = np.array([v for *_, v in ref["grad_norms"]])
    r_gpu, c_gpu = report("sampled grads vs fp64 oracle", got, want_f)
    r_mir, c_mir = report("mirror oracle vs fp64 oracle", want_m, want_f)
    report("sampled grads vs mirror oracle", got, want_m)
    assert r_gpu <= 1.25 * r_mir and c_gpu >= c_mir - 1e-3, (r_gpu, r_mir, c_gpu, c_mir)
    e_gpu = np.max(np.abs(gn - wn_f) / wn_f)
    e_mir = np.max(np.abs(wn_m - wn_f) / wn_f)
    print(f"grad norms: max rel vs fp64 {e_gpu:.3e} (mirror {e_mir:.3e}), vs mirror "
          f"{np.max(np.abs(gn - wn_m) / wn_m):.3e}", flush=True)
    assert e_gpu <= 1.25 * e_mir, (e_gpu, e_mir)


@pytest.mark.timeout(900)
def test_full_8b_step_seq4096(q, stack8b):
    """Seq 4096: streamed == resident bitwise, layers 0 and 31 against the
    oracle at the gradient bar, the loss against the golden value."""
    cfg, store, res = stack8b
    S = 4096
    ids = torch.from_numpy(synth.token_ids(cfg, 1, S, seed=42)).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    print("8B step at seq 4096, streamed (captured)", flush=True)
    s = _sft_run(q, cfg, store, res, ids, lora, q.QLS_STREAMED, capture=True)
    print("8B step at seq 4096, resident", flush=True)
    r = _sft_run(q, cfg, store, res, ids, lora, q.QLS_RESIDENT, capture=False)
    assert np.array_equal(s["loss"], r["loss"])
    assert np.array_equal(s["ck"], r["ck"])
    assert np.array_equal(bits(s["grads"]), bits(r["grads"]))
    del r
    print(f"seq-4096 loss {s['hl']:.6f}", flush=True)
    if os.path.exists(GOLDEN4096):
        gold = json.load(open(GOLDEN4096))["loss"]
        print(f"golden (mirror oracle) loss {gold:.6f}", flush=True)
        assert abs(s["hl"] - gold) <= 1e-3 * abs(gold), (s["hl"], gold)
    n = cpu_share()
    _per_layer_check(cfg, [0, cfg.L - 1], s["ck"], s["cap"], s["grads"], synth.lora_init(cfg), 1, S,
                     2, max(1, n // 2))
    if not os.path.exists(GOLDEN4096):
        pytest.skip("golden loss not generated (tests/golden/make_golden_8b.py --task sft --seq 4096 --loss-only)")


@pytest.mark.timeout(900)
def test_full_8b_dpo(q, stack8b):
    cfg, store, res = stack8b
    S, P, beta = 512, 128, 0.1
    c, r = synth.dpo_pair(cfg, S, P)
    ids2 = torch.from_numpy(np.stack([c, r])).cuda()
    chosen, rejected = ids2[0].contiguous(), ids2[1].contiguous()
    lora_np = synth.lora_init(cfg)
    lora = torch.from_numpy(synth.pack_lora(cfg, lora_np)).cuda()
    runs = {}
    for mode in (q.QLS_STREAMED, q.QLS_RESIDENT):
        print(f"8B DPO step mode {mode}", flush=True)
        sess = q.Session(store, *res, max_tokens=2 * S, max_seq=S, mode=mode)
        cap = None
        if mode == q.QLS_STREAMED:
            cap = torch.full(((cfg.L + 1) * 2 * S * cfg.d,), float("nan"), device="cuda")
            sess.capture_grads(cap)
            ref = torch.empty(2, device="cuda")
            sess.logprobs(ids2, P, None, ref)
        grads = torch.full_like(lora, float("nan"))
        loss = torch.empty(1, device="cuda")
        aux = torch.empty(4, device="cuda")
        hl = sess.dpo_step(chosen, rejected, P, beta, lora, grads, loss, aux, host_loss=True)
        runs[mode] = {"hl": hl, "loss": bits(loss), "aux": bits(aux), "grads": grads.cpu(),
                      "ck": bits(sess.checkpoints(2 * S))}
        if cap is not None:
            runs[mode]["cap"] = cap.view(cfg.L + 1, 2 * S, cfg.d).cpu().numpy()
            runs[mode]["ref"] = bits(ref)
        sess.close()
    s, rr = runs[q.QLS_STREAMED], runs[q.QLS_RESIDENT]
    assert np.array_equal(s["loss"], rr["loss"])
    assert np.array_equal(s["aux"], rr["aux"])
    assert np.array_equal(s["ck"], rr["ck"])
    assert np.array_equal(bits(s["grads"]), bits(rr["grads"]))
    assert np.array_equal(s["aux"][2:], s["ref"])               # fused reference == standalone pass
    assert np.all(np.isfinite(s["grads"].numpy()))
    aux = s["aux"].view(np.float32).astype(np.float64)
    z = beta * ((aux[0] - aux[2]) - (aux[1] - aux[3]))
    print(f"8B DPO loss {s['hl']:.7f}, pi {aux[:2]}, rho {aux[2:]}, z {z:.6f}", flush=True)
    # Every layer of the step's backward at the gradient bar, given its inputs.
    n = cpu_share()
    _per_layer_check(cfg, [0, cfg.L // 2, cfg.L - 1], s["ck"], s["cap"], s["grads"], lora_np, 2, S, 3,
                     max(1, n // 3))
    if not (os.path.exists(GOLDEN_DPO) and os.path.exists(GOLDEN_DPO64)):
        pytest.skip("golden values not generated (tests/golden/make_golden_8b.py --task dpo [--prec fp64])")
    mir, f64 = json.load(open(GOLDEN_DPO)), json.load(open(GOLDEN_DPO64))
    for name, gold in (("mirror", mir), ("fp64", f64)):
        print(f"golden ({name} oracle): loss {gold['loss']:.7f}, pi {gold['pi']}, rho {gold['ref']}, "
              f"z {gold['z']:.6f}", flush=True)
        # The summed response log-likelihoods: within 1e-3 of both oracles.
        for got, want in zip(aux, gold["pi"] + gold["ref"]):
            assert abs(got - want) <= 1e-3 * abs(want), (name, got, want)
    # The loss is a function of z = beta ((pi_c - rho_c) - (pi_r - rho_r)), a
    # difference of ~4800-nat sums that the adapters (B ~ N(0, 1e-3)) move by
    # well under a nat: bf16 rounding through 32 layers moves each sum by about
    # a nat, so the mirror-precision oracle itself lands 0.09 (13%) from the
    # fp64 oracle's loss.  As for the SFT gradients, the GPU must be as close to
    # the fp64 oracle as the mirror oracle is (25% slack), in z and in the loss.
    dz_gpu, dz_mir = abs(z - f64["z"]), abs(mir["z"] - f64["z"])
    dl_gpu, dl_mir = abs(s["hl"] - f64["loss"]), abs(mir["loss"] - f64["loss"])
    print(f"|z - z_fp64|: GPU {dz_gpu:.4f}, mirror oracle {dz_mir:.4f}; |loss - loss_fp64|: GPU {dl_gpu:.4f}, "
          f"mirror oracle {dl_mir:.4f}", flush=True)
    assert dz_gpu <= 1.25 * dz_mir and dl_gpu <= 1.25 * dl_mir, (dz_gpu, dz_mir, dl_gpu, dl_mir)
    # Whole-stack gradients: the same propagation reading.
    per = synth.unpack_lora(cfg, s["grads"].numpy())
    got = np.array([per[l][om.NAMES[m]][w].reshape(-1)[i] for l, m, w, i, _ in mir["samples"]])
    want_m = np.array([v for *_, v in mir["samples"]])
    want_f = np.array([v for *_, v in f64["samples"]])
    r_gpu, c_gpu = report("DPO sampled grads vs fp64 oracle", got, want_f)
    r_mir, c_mir = report("mirror oracle vs fp64 oracle", want_m, want_f)
    report("DPO sampled grads vs mirror oracle", got, want_m)
    assert r_gpu <= 1.25 * r_mir and c_gpu >= c_mir - 2e-3, (r_gpu, r_mir, c_gpu, c_mir)


def test_full_8b_dpo_b_zero(q, stack8b):
    cfg, store, res = stack8b
    S, P, beta = 512, 128, 0.1
    c, r = synth.dpo_pair(cfg, S, P)
    ids2 = torch.from_numpy(np.stack([c, r])).cuda()
    sess = q.Session(store, *res, max_tokens=2 * S, max_seq=S)
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=0.0))).cuda()
    grads = torch.full_like(lora, float("nan"))
    loss = torch.empty(1, device="cuda")
    aux = torch.empty(4, device="cuda")
    hl = sess.dpo_step(ids2[0].contiguous(), ids2[1].contiguous(), P, beta, lora, grads, loss, aux,
                       host_loss=True)
    a = bits(aux)
    assert bool(torch.isfinite(grads).all())
    assert np.array_equal(a[:2], a[2:]) and hl == np.float32(math.log(2.0))
    sess.close()
