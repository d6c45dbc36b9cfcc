"""The disk tier on the GPU: a store whose layers spill to a file streams to
the same bits as the pinned store, through the C ABI.

  * SFT with every layer on disk, and with half of them, equals the pinned
    resident run bit for bit (loss, layer-input checkpoints, LoRA gradients),
    over two consecutive steps (the second reuses the slots across the step
    boundary), also with slots poisoned on release and with copy / compute
    delays injected;
  * a resident session over the tiered store equals it too;
  * the fused DPO step over the tiered store equals the pinned streamed one;
  * layer-load counts are those of the pinned store; every load of a disk
    layer is a file read (read-aheads may add reads, never bytes per read).
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import bits
from tests.test_gpu_step import _run_sft

pytestmark = pytest.mark.gpu
CFG = synth.scaled(synth.TINY, L=6)


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _fill(store, cfg):
    for l in range(cfg.L):
        na, nm = synth.layer_norms(cfg, l, True)
        store.set_layer_fp32(l, synth.base_layer(cfg, l), na, nm)
    return store


@pytest.fixture(scope="module")
def stores(q, tmp_path_factory):
    d = tmp_path_factory.mktemp("disk")
    res = (synth.embedding(CFG).cuda(), synth.lm_head(CFG).cuda(), synth.final_norm(CFG, True).cuda())
    pinned = _fill(q.Store(CFG, absmax="dq8"), CFG)
    all_disk = _fill(q.Store(CFG, absmax="dq8", ram_layers=0, disk_path=d / "all.bin"), CFG)
    half = _fill(q.Store(CFG, absmax="dq8", ram_layers=3, disk_path=d / "half.bin"), CFG)
    yield {"pinned": pinned, "disk": all_disk, "half": half}, res
    for s in (pinned, all_disk, half):
        s.close()


def test_disk_tier_streams_the_same_bits(q, stores):
    st, res = stores
    ids = synth.token_ids(CFG, 1, 64, seed=3)
    lora = synth.lora_init(CFG, b_std=0.01)
    runs = [("pinned-resident", "pinned", q.QLS_RESIDENT, 0), ("disk-streamed", "disk", q.QLS_STREAMED, 0),
            ("half-streamed", "half", q.QLS_STREAMED, 0),
            ("disk-poison", "disk", q.QLS_STREAMED, q.DBG_POISON_ON_RELEASE),
            ("half-delays", "half", q.QLS_STREAMED, q.DBG_COPY_DELAY | q.DBG_COMPUTE_DELAY),
            ("disk-resident", "disk", q.QLS_RESIDENT, 0)]
    out = {}
    for name, key, mode, flags in runs:
        print(f"run {name}", flush=True)
        sess = q.Session(st[key], *res, max_tokens=64, max_seq=64, mode=mode)
        sess.debug(flags, 2000 if flags & q.DBG_COPY_DELAY else 0)
        got = []
        for step in range(2):
            sess.reset_stats()
            hl, loss, grads = _run_sft(q, sess, CFG, ids, lora)
            got.append((bits(loss), bits(grads), bits(sess.checkpoints(64))))
            s = sess.stats()
            if mode == q.QLS_STREAMED:
                pinned_layers = st[key].ram_layers
                if flags == 0:
                    assert s["layer_loads"] == (2 * CFG.L - 2 if step == 0 else 2 * CFG.L - 4)
                if pinned_layers < CFG.L:
                    assert s["disk_reads"] >= 1 and s["disk_bytes"] == s["disk_reads"] * st[key].record_bytes
        for a, b in zip(got[0], got[1]):
            assert np.array_equal(a, b), name
        out[name] = got[0]
        sess.close()
    ref = out["pinned-resident"]
    for name in out:
        assert np.array_equal(out[name][0], ref[0]), name      # loss
        assert np.array_equal(out[name][2], ref[2]), name      # checkpoints
        assert np.array_equal(out[name][1], ref[1]), name      # gradients


def test_disk_tier_dpo_equals_pinned(q, stores):
    st, res = stores
    c, r = synth.dpo_pair(CFG, 64, 16)
    lora = torch.from_numpy(synth.pack_lora(CFG, synth.lora_init(CFG, b_std=0.02))).cuda()
    out = {}
    for key in ("pinned", "disk"):
        sess = q.Session(st[key], *res, max_tokens=128, max_seq=64)
        grads = torch.empty_like(lora)
        loss = torch.empty(1, device="cuda")
        aux = torch.empty(4, device="cuda")
        sess.dpo_step(torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda(), 16, 0.1, lora, grads, loss, aux)
        torch.cuda.synchronize()
        out[key] = (bits(loss), bits(grads), bits(aux), sess.stats()["layer_loads"])
        sess.close()
    for a, b in zip(out["pinned"], out["disk"]):
        assert np.array_equal(a, b)
