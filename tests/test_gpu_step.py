"""GPU parity of the streamed step on a tiny Llama-style stack, through the C ABI.

  * SFT loss within 1e-3 relative of the oracle, LoRA gradients within 1e-2
    relative L2 and cosine >= 0.999 (whole vector and per matrix);
  * streamed == resident, bit for bit: loss, every layer-input checkpoint
    (the forward question) and every dA / dB (the gradient question), also
    with slots poisoned on release and with copy / compute delays injected
    (page "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU? ...", sections "Did a
    correctness bug invalidate ..." and "The gradient bug also reveals ...");
  * adapters-disabled log-probs equal the fused DPO reference, bit for bit;
  * layer-load counts: 2L - 2 per SFT step, 3L - 2 for a separate reference
    sweep plus a policy step (page "Soup ... radar note", section "In detail":
    1.52x for DPO at 32 layers);
  * the same parity and streamed == resident checks on a store with
    double-quantised absmax (8-bit codes + one float32 scale per 256 blocks).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from tests.gpu_util import bits, f32, report, same_values
from tests.helpers import cosine, rel_l2

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _setup(q, cfg, perturbed=True, absmax="f32"):
    store = q.Store(cfg, absmax=absmax)
    layers = []
    for l in range(cfg.L):
        ws = synth.base_layer(cfg, l)
        na, nm = synth.layer_norms(cfg, l, perturbed)
        store.set_layer_fp32(l, ws, na, nm)
        layers.append(om.dequant_layer(cfg, ws, na.float().numpy(), nm.float().numpy(), absmax=absmax))
    emb, lm, fn = synth.embedding(cfg), synth.lm_head(cfg), synth.final_norm(cfg, perturbed)
    model = om.Model(cfg, layers, emb.float().numpy(), lm.float().numpy(), fn.float().numpy())
    return store, model, (emb.cuda(), lm.cuda(), fn.cuda())


@pytest.fixture(scope="module")
def tiny(q):
    cfg = synth.TINY
    store, model, res = _setup(q, cfg)
    return cfg, store, model, res


def _flat_oracle_grads(cfg, og):
    return np.concatenate([np.concatenate([og[l][n][0].ravel(), og[l][n][1].ravel()])
                           for l in range(cfg.L) for n in om.NAMES])


def _run_sft(q, sess, cfg, ids, lora):
    d_lora = torch.from_numpy(synth.pack_lora(cfg, lora)).cuda()
    grads = torch.full_like(d_lora, float("nan"))
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    hl = sess.sft_step(torch.from_numpy(ids).cuda(), d_lora, grads, loss, host_loss=True)
    torch.cuda.synchronize()
    return hl, loss, grads


def test_sft_matches_oracle(q, tiny):
    cfg, store, model, res = tiny
    ids = synth.token_ids(cfg, 1, 64)
    lora = synth.lora_init(cfg)
    sess = q.Session(store, *res, max_tokens=64, max_seq=64)
    hl, loss, grads = _run_sft(q, sess, cfg, ids, lora)
    ol, og, aux = om.sft_step(cfg, PM, model, lora, ids)
    print(f"loss gpu={hl:.7f} oracle={ol:.7f}", flush=True)
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    ck = sess.checkpoints(64)
    for l in range(cfg.L + 1):
        r, _ = report(f"x_{l}", f32(ck[l]), aux["xs"][l])
        assert r <= 1e-2
    got = grads.cpu().numpy()
    r, c = report("grads", got, _flat_oracle_grads(cfg, og))
    assert r <= 1e-2 and c >= 0.999
    per = synth.unpack_lora(cfg, got)
    for l in range(cfg.L):
        for n in om.NAMES:
            for w in range(2):
                rr, cc = rel_l2(per[l][n][w], og[l][n][w]), cosine(per[l][n][w], og[l][n][w])
                assert rr <= 1e-2 and cc >= 0.999, (l, n, w, rr, cc)
    sess.close()


def test_sft_two_sequences_matches_oracle(q, tiny):
    cfg, store, model, res = tiny
    ids = synth.token_ids(cfg, 2, 48, seed=17)
    lora = synth.lora_init(cfg, b_std=0.01)
    sess = q.Session(store, *res, max_tokens=96, max_seq=48, ce_chunk=384)
    hl, _, grads = _run_sft(q, sess, cfg, ids, lora)
    ol, og, _ = om.sft_step(cfg, PM, model, lora, ids)
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    r, c = report("grads B=2", grads.cpu().numpy(), _flat_oracle_grads(cfg, og))
    assert r <= 1e-2 and c >= 0.999
    sess.close()


# One 4096-wide layer with a small vocabulary at 4096 tokens: the LM head's
# dh = dlogits W product (4096 x 4096 outputs, two vocabulary chunks of 1024)
# runs on the 256 x 256 kernel with the bf16 weight read row-major and
# transposed in LDS, written by the first chunk and accumulated by the second.
HEAD_WIDE = synth.ModelCfg(L=1, d=4096, H=8, KV=2, hd=128, I=512, V=2048, eps=1e-5,
                           theta=500000.0, r=8, alpha=16.0)


def test_lm_head_on_large_tiles_matches_oracle(q):
    cfg = HEAD_WIDE
    store, model, res = _setup(q, cfg)
    ids = synth.token_ids(cfg, 1, 4096, seed=23)
    lora = synth.lora_init(cfg, b_std=0.01)
    sess = q.Session(store, *res, max_tokens=4096, max_seq=4096, ce_chunk=1024)
    hl, _, grads = _run_sft(q, sess, cfg, ids, lora)
    sess.close()
    print("oracle step at 4096 tokens", flush=True)
    ol, og, _ = om.sft_step(cfg, PM, model, lora, ids)
    print(f"loss gpu={hl:.7f} oracle={ol:.7f}", flush=True)
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    r, c = report("grads wide head", grads.cpu().numpy(), _flat_oracle_grads(cfg, og))
    assert r <= 1e-2 and c >= 0.999


def test_b_zero_gives_zero_dA(q, tiny):
    cfg, store, model, res = tiny
    sess = q.Session(store, *res, max_tokens=64, max_seq=64)
    _, _, grads = _run_sft(q, sess, cfg, synth.token_ids(cfg, 1, 64), synth.lora_init(cfg, b_std=0.0))
    per = synth.unpack_lora(cfg, grads.cpu().numpy())
    for l in range(cfg.L):
        for n in om.NAMES:
            assert not np.any(per[l][n][0]), (l, n)
            assert np.any(per[l][n][1]), (l, n)
    sess.close()


def _deep_cfg():
    return synth.scaled(synth.TINY, L=6)


@pytest.fixture(scope="module")
def deep(q):
    cfg = _deep_cfg()
    store, model, res = _setup(q, cfg)
    return cfg, store, model, res


def test_streamed_equals_resident_bitwise(q, deep):
    cfg, store, _, res = deep
    ids = synth.token_ids(cfg, 1, 64, seed=3)
    lora = synth.lora_init(cfg, b_std=0.01)
    out = {}
    for name, mode, flags in [("resident", q.QLS_RESIDENT, 0), ("streamed", q.QLS_STREAMED, 0),
                              ("poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE),
                              ("delays", q.QLS_STREAMED, q.DBG_COPY_DELAY | q.DBG_COMPUTE_DELAY),
                              ("compute-delay", q.QLS_STREAMED, q.DBG_COMPUTE_DELAY),
                              ("stream-fence", q.QLS_STREAMED, q.DBG_STREAM_FENCE),
                              ("stream-fence-delays", q.QLS_STREAMED,
                               q.DBG_STREAM_FENCE | q.DBG_COPY_DELAY | q.DBG_COMPUTE_DELAY)]:
        print(f"run {name}", flush=True)
        sess = q.Session(store, *res, max_tokens=64, max_seq=64, mode=mode)
        sess.debug(flags, 2000 if flags & (q.DBG_COPY_DELAY | q.DBG_COMPUTE_DELAY) else 0)
        for _ in range(2):                        # the second step starts with layers 0 and 1 resident
            hl, loss, grads = _run_sft(q, sess, cfg, ids, lora)
        out[name] = (bits(loss), bits(grads), bits(sess.checkpoints(64)))
        sess.close()
    for name in ("streamed", "poison", "delays", "compute-delay", "stream-fence", "stream-fence-delays"):
        assert np.array_equal(out[name][0], out["resident"][0]), name           # loss
        assert np.array_equal(out[name][2], out["resident"][2]), name           # forward question
        assert np.array_equal(out[name][1], out["resident"][1]), name           # gradient question
    assert np.all(np.isfinite(out["resident"][1].view(np.float32)))


def test_dpo_streamed_equals_resident_bitwise(q, deep):
    """The fused reference pass reads every resident layer twice before the
    slot's code parts are released; the first copy of each sweep then goes in
    parts (on 6 layers: layer 2 forward, layer 3 backward)."""
    cfg, store, _, res = deep
    c, r = synth.dpo_pair(cfg, 64, 16)
    c, r = torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda()
    d_lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=0.01))).cuda()
    out = {}
    for name, mode, flags in [("resident", q.QLS_RESIDENT, 0), ("streamed", q.QLS_STREAMED, 0),
                              ("compute-delay", q.QLS_STREAMED, q.DBG_COMPUTE_DELAY),
                              ("poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE)]:
        print(f"dpo run {name}", flush=True)
        sess = q.Session(store, *res, max_tokens=128, max_seq=64, mode=mode)
        sess.debug(flags, 2000 if flags & q.DBG_COMPUTE_DELAY else 0)
        grads = torch.full_like(d_lora, float("nan"))
        loss = torch.empty(1, dtype=torch.float32, device="cuda")
        for _ in range(2):
            sess.dpo_step(c, r, 16, 0.1, d_lora, grads, loss)
        torch.cuda.synchronize()
        out[name] = (bits(loss), bits(grads))
        sess.close()
    for name in ("streamed", "compute-delay", "poison"):
        assert np.array_equal(out[name][0], out["resident"][0]), name
        assert np.array_equal(out[name][1], out["resident"][1]), name
    assert np.all(np.isfinite(out["resident"][1].view(np.float32)))


def test_layer_load_counts(q, deep):
    cfg, store, _, res = deep
    L = cfg.L
    ids = torch.from_numpy(synth.token_ids(cfg, 1, 64)).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    grads = torch.empty_like(lora)
    loss = torch.empty(1, device="cuda")
    sess = q.Session(store, *res, max_tokens=128, max_seq=64)
    sess.sft_step(ids, lora, grads, loss)
    st = sess.stats()
    assert st["layer_loads"] == 2 * L - 2 and st["h2d_bytes"] == (2 * L - 2) * store.record_bytes
    sess.reset_stats()
    sess.sft_step(ids, lora, grads, loss)       # layers 0 and 1 are still resident
    assert sess.stats()["layer_loads"] == 2 * L - 4
    sess.debug(q.DBG_NO_REUSE)
    sess.reset_stats()
    sess.sft_step(ids, lora, grads, loss)
    sft = sess.stats()["layer_loads"]
    assert sft == 2 * L - 2
    seq = torch.empty(1, device="cuda")
    sess.reset_stats()
    sess.logprobs(ids, 16, None, seq)            # a separate reference sweep
    ref = sess.stats()["layer_loads"]
    assert ref == L
    # fused DPO streams like SFT; a separate reference sweep would cost 3L - 2
    assert (ref + sft) == 3 * L - 2
    c, r = synth.dpo_pair(cfg, 64, 16)
    sess.reset_stats()
    sess.dpo_step(torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda(), 16, 0.1, lora, grads, loss)
    assert sess.stats()["layer_loads"] == 2 * L - 2
    sess.close()


def test_logprobs_and_dpo_match_oracle(q, tiny):
    cfg, store, model, res = tiny
    S, P, beta = 64, 16, 0.1
    c, r = synth.dpo_pair(cfg, S, P)
    lora = synth.lora_init(cfg, b_std=0.02)
    d_lora = torch.from_numpy(synth.pack_lora(cfg, lora)).cuda()
    sess = q.Session(store, *res, max_tokens=2 * S, max_seq=S)
    ids2 = torch.from_numpy(np.stack([c, r])).cuda()
    ref = torch.empty(2, device="cuda")
    tok = torch.empty(2, S, device="cuda")
    sess.logprobs(ids2, P, None, ref, tok)
    grads = torch.empty_like(d_lora)
    loss = torch.empty(1, device="cuda")
    aux = torch.empty(4, device="cuda")
    hl = sess.dpo_step(ids2[0].contiguous(), ids2[1].contiguous(), P, beta, d_lora, grads, loss, aux,
                       host_loss=True)
    torch.cuda.synchronize()
    # the fused reference equals the standalone adapters-disabled pass, bit for bit
    assert np.array_equal(bits(aux)[2:], bits(ref))
    oref, _ = om.seq_logprobs(cfg, PM, model, None, np.stack([c, r]), P)
    report("ref logp", f32(ref), oref)
    assert np.allclose(f32(ref), oref, rtol=1e-3)
    ol, og, oaux = om.dpo_step(cfg, PM, model, lora, c, r, P, beta)
    print(f"dpo loss gpu={hl:.7f} oracle={ol:.7f} z={oaux['z']:.5f}", flush=True)
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    rr, cc = report("dpo grads", grads.cpu().numpy(), _flat_oracle_grads(cfg, og))
    assert rr <= 1e-2 and cc >= 0.999
    sess.close()


def test_dpo_b_zero_is_ln2(q, tiny):
    cfg, store, _, res = tiny
    c, r = synth.dpo_pair(cfg, 64, 16)
    d_lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=0.0))).cuda()
    sess = q.Session(store, *res, max_tokens=128, max_seq=64)
    grads = torch.empty_like(d_lora)
    loss = torch.empty(1, device="cuda")
    aux = torch.empty(4, device="cuda")
    hl = sess.dpo_step(torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda(), 16, 0.1, d_lora, grads, loss,
                       aux, host_loss=True)
    a = f32(aux)
    assert same_values(a[:2], a[2:])                  # policy == reference when B = 0
    assert hl == np.float32(np.log(2.0))
    sess.close()


def test_bad_token_id_is_reported(q, tiny):
    cfg, store, _, res = tiny
    sess = q.Session(store, *res, max_tokens=64, max_seq=64)
    ids = synth.token_ids(cfg, 1, 64)
    ids[0, 5] = cfg.V + 3
    with pytest.raises(q.QlsError) as e:
        _run_sft(q, sess, cfg, ids, synth.lora_init(cfg))
    assert e.value.code == q.QLS_EINVAL
    sess.stats()                                  # reported once, then cleared
    with pytest.raises(q.QlsError):
        _run_sft(q, sess, cfg, synth.token_ids(cfg, 1, 80), synth.lora_init(cfg))   # S > max_seq
    # Without a host loss the flag stays raised until qls_session_stats reports it.
    d_lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    grads = torch.empty_like(d_lora)
    loss = torch.empty(1, device="cuda")
    sess.sft_step(torch.from_numpy(ids).cuda(), d_lora, grads, loss)
    sess.sft_step(torch.from_numpy(synth.token_ids(cfg, 1, 64)).cuda(), d_lora, grads, loss)
    with pytest.raises(q.QlsError) as e:
        sess.stats()
    assert e.value.code == q.QLS_EINVAL
    sess.stats()
    hl, _, _ = _run_sft(q, sess, cfg, synth.token_ids(cfg, 1, 64), synth.lora_init(cfg))
    assert np.isfinite(hl)
    sess.close()


def test_stats_exposed_copy_and_peak_workspace(q, deep):
    cfg, store, _, res = deep
    sess = q.Session(store, *res, max_tokens=128, max_seq=64, timing=True)
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    grads = torch.empty_like(lora)
    loss = torch.empty(1, device="cuda")
    sess.sft_step(torch.from_numpy(synth.token_ids(cfg, 1, 32)).cuda(), lora, grads, loss)
    st = sess.stats()
    assert 0 < st["peak_ws_bytes"] < st["ws_bytes"]
    assert st["copy_ms"] > 0 and abs(st["exposed_copy_ms"] - (st["copy_ms"] - st["overlap_ms"])) < 1e-9
    small = st["peak_ws_bytes"]
    sess.sft_step(torch.from_numpy(synth.token_ids(cfg, 2, 64)).cuda(), lora, grads, loss)
    st = sess.stats()
    assert small < st["peak_ws_bytes"] <= st["ws_bytes"]
    run = q.RunCfg(q.QLS_STREAMED, 128, 64, 0, 1)
    assert st["peak_ws_bytes"] == q.qls_workspace_bytes(store.h, run)
    sess.reset_stats()
    assert sess.stats()["peak_ws_bytes"] == 0
    sess.close()


def test_recompute_all_is_bit_identical(q, deep):
    """The two ends of the backward sweep reuse forward intermediates instead
    of recomputing them (the last layer's at the turn, layer 0's saved copy);
    recomputing every layer must give the same bits: loss, checkpoints and
    every gradient, for SFT and DPO, streamed and resident."""
    cfg, store, _, res = deep
    ids = torch.from_numpy(synth.token_ids(cfg, 1, 64, seed=3)).cuda()
    c, r = synth.dpo_pair(cfg, 64, 16)
    c, r = torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg, b_std=0.01))).cuda()
    out = {}
    for mode in (q.QLS_STREAMED, q.QLS_RESIDENT):
        for flags in (0, q.DBG_RECOMPUTE_ALL):
            sess = q.Session(store, *res, max_tokens=128, max_seq=64, mode=mode)
            sess.debug(flags)
            grads = torch.full_like(lora, float("nan"))
            loss = torch.empty(1, device="cuda")
            sess.sft_step(ids, lora, grads, loss)
            sft = (bits(loss), bits(grads), bits(sess.checkpoints(64)))
            aux = torch.empty(4, device="cuda")
            sess.dpo_step(c, r, 16, 0.1, lora, grads, loss, aux)
            out[mode, flags] = sft + (bits(loss), bits(aux), bits(grads))
            sess.close()
    want = out[q.QLS_RESIDENT, 0]
    for key, got in out.items():
        for a, b in zip(got, want):
            assert np.array_equal(a, b), key
    assert np.all(np.isfinite(want[1].view(np.float32)))


def test_gradient_capture(q, tiny):
    """The capture hook adds copies only (gradients, loss and checkpoints equal
    an uncaptured step bit for bit); entry l holds dL/dx_l: entry 0 against the
    oracle's dL/dx_0, and every layer of the step against the oracle given that
    layer's checkpoint and captured incoming gradient."""
    from tests.layer_oracle import run_layers
    cfg, store, model, res = tiny
    ids = synth.token_ids(cfg, 1, 64)
    lora = synth.lora_init(cfg)
    d_lora = torch.from_numpy(synth.pack_lora(cfg, lora)).cuda()
    runs = []
    for capture in (False, True):
        sess = q.Session(store, *res, max_tokens=64, max_seq=64)
        cap = torch.full(((cfg.L + 1) * 64 * cfg.d,), float("nan"), device="cuda")
        if capture:
            small = torch.empty((cfg.L + 1) * 64 * cfg.d - 1, device="cuda")
            sess.capture_grads(small)
            with pytest.raises(q.QlsError) as e:
                _run_sft(q, sess, cfg, ids, lora)
            assert e.value.code == q.QLS_EINVAL
            sess.capture_grads(cap)
        hl, loss, grads = _run_sft(q, sess, cfg, ids, lora)
        runs.append((bits(loss), bits(grads), bits(sess.checkpoints(64)), cap.view(cfg.L + 1, 64, cfg.d).cpu(),
                     sess.checkpoints(64).float().cpu().numpy(), grads.cpu().numpy()))
        sess.close()
    for a, b in zip(runs[0][:3], runs[1][:3]):
        assert np.array_equal(a, b)
    cap, ck, grads = runs[1][3].numpy(), runs[1][4], runs[1][5]
    assert np.all(np.isfinite(cap))
    _, _, aux = om.sft_step(cfg, PM, model, lora, ids)
    rr, cc = report("dL/dx_0", cap[0], aux["g0"])
    assert rr <= 1e-2 and cc >= 0.999
    jobs = [(cfg, l, ck[l], cap[l + 1], lora[l], 1, 64, "f32", True) for l in range(cfg.L)]
    res_o = run_layers(jobs, workers=2, threads=2)
    per = synth.unpack_lora(cfg, grads)
    for l in range(cfg.L):
        out, g_in, og = res_o[l]
        for name, got, want in [("out", ck[l + 1], out), ("dL/dx", cap[l], g_in)] + [
                (f"{n}.{'AB'[w]}", per[l][n][w], og[n][w]) for n in om.NAMES for w in range(2)]:
            rr, cc = rel_l2(got, want), cosine(got, want)
            assert rr <= 1e-2 and cc >= 0.999, (l, name, rr, cc)


def test_degenerate_sizes_are_refused(q, tiny):
    """No next-token target (S = 1), more tokens than the workspace holds, and
    an empty batch are refused before any launch; the session stays usable."""
    cfg, store, _, res = tiny
    sess = q.Session(store, *res, max_tokens=64, max_seq=64)
    lora = synth.lora_init(cfg)
    for B, S in [(1, 1), (2, 48), (0, 16)]:
        with pytest.raises(q.QlsError) as e:
            _run_sft(q, sess, cfg, synth.token_ids(cfg, B, S), lora)
        assert e.value.code == q.QLS_EINVAL, (B, S)
    hl, _, grads = _run_sft(q, sess, cfg, synth.token_ids(cfg, 1, 64), lora)
    assert np.isfinite(hl) and np.all(np.isfinite(grads.cpu().numpy()))
    sess.close()


def test_workspace_too_small_is_rejected(q, tiny):
    cfg, store, _, res = tiny
    run = q.RunCfg(q.QLS_STREAMED, 64, 64, 0, 0)
    need = q.qls_workspace_bytes(store.h, run)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with pytest.raises(q.QlsError) as e:
        q.qls_session_create(store.h, run, ws, need - 256, s, s, *res)
    assert e.value.code == q.QLS_ENOMEM


# ---------------------------------------------------------------- double-quantised absmax store
@pytest.fixture(scope="module")
def tiny_dq(q):
    cfg = synth.TINY
    store, model, res = _setup(q, cfg, absmax="dq8")
    return cfg, store, model, res


def test_dq_store_holds_the_oracle_double_quant(q, tiny_dq):
    from oracle import nf4
    cfg, store, _, _ = tiny_dq
    assert store.record_bytes < q.qls_layer_record_bytes(q.model_cfg(cfg))
    rec = store.layer(1)
    for m, w in enumerate(synth.base_layer(cfg, 1)):
        codes, amax = nf4.quantize(w)
        q8, sc = nf4.double_quant(amax)
        assert np.array_equal(rec["codes"][m], codes)
        assert np.array_equal(rec["absmax_q8"][m], q8)
        assert np.array_equal(rec["absmax_scale"][m].view(np.uint32), sc.view(np.uint32))


def test_dq_sft_matches_oracle(q, tiny_dq):
    cfg, store, model, res = tiny_dq
    ids = synth.token_ids(cfg, 1, 64)
    lora = synth.lora_init(cfg)
    sess = q.Session(store, *res, max_tokens=64, max_seq=64)
    hl, loss, grads = _run_sft(q, sess, cfg, ids, lora)
    ol, og, _ = om.sft_step(cfg, PM, model, lora, ids)
    print(f"dq8 loss gpu={hl:.7f} oracle={ol:.7f}", flush=True)
    assert abs(hl - ol) <= 1e-3 * abs(ol)
    r, c = report("dq8 grads", grads.cpu().numpy(), _flat_oracle_grads(cfg, og))
    assert r <= 1e-2 and c >= 0.999
    sess.close()


def test_dq_streamed_equals_resident_bitwise(q):
    cfg = _deep_cfg()
    store, _, res = _setup(q, cfg, absmax="dq8")
    ids = synth.token_ids(cfg, 1, 64, seed=3)
    lora = synth.lora_init(cfg, b_std=0.01)
    out = {}
    for name, mode, flags in [("resident", q.QLS_RESIDENT, 0), ("streamed", q.QLS_STREAMED, 0),
                              ("poison", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE),
                              ("no-reuse", q.QLS_STREAMED, q.DBG_NO_REUSE)]:
        print(f"dq8 run {name}", flush=True)
        sess = q.Session(store, *res, max_tokens=64, max_seq=64, mode=mode)
        sess.debug(flags)
        for _ in range(2):                        # the second step reuses slots and expansions
            hl, loss, grads = _run_sft(q, sess, cfg, ids, lora)
        out[name] = (bits(loss), bits(grads), bits(sess.checkpoints(64)))
        st = sess.stats()
        if mode == q.QLS_STREAMED:
            assert st["h2d_bytes"] == st["layer_loads"] * store.record_bytes
        sess.close()
    for name in ("streamed", "poison", "no-reuse"):
        for a, b in zip(out[name], out["resident"]):
            assert np.array_equal(a, b), name


def test_unsupported_session_configs_are_refused(q, tiny):
    """A resident tensor off the 256-byte alignment the kernels assume, and a
    hidden size above the RMSNorm-backward kernel's 8192, are refused before
    any launch."""
    cfg, store, _, res = tiny
    emb, lm, fn = res
    off = torch.empty(emb.numel() + 64, dtype=torch.bfloat16, device="cuda")[8:8 + emb.numel()].view_as(emb)
    run = q.RunCfg(q.QLS_STREAMED, 64, 64, 0, 0)
    need = q.qls_workspace_bytes(store.h, run)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with pytest.raises(q.QlsError) as e:
        q.qls_session_create(store.h, run, ws, need, s, s, off, lm, fn)
    assert e.value.code == q.QLS_EINVAL
    wide = synth.scaled(cfg, L=1, d=8448, H=66, KV=66, hd=128, I=256)
    big = q.Store(wide)
    with pytest.raises(q.QlsError) as e:
        q.qls_workspace_bytes(big.h, run)
    assert e.value.code == q.QLS_EINVAL
    big.close()
