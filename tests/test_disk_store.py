"""Disk tier of the layer store on the host (no GPU): a store whose layers all
live in the file (ram_layers = 0) holds, per layer, exactly the oracle's NF4
codes and absmax (float32, or the double-quantised 8-bit codes and group
scales) and the norms; the file has one 4096-byte-aligned slot per layer and
goes away with the store; bad arguments and file errors are reported."""
import dataclasses
import os

import numpy as np
import pytest

import synth
from oracle import nf4

TINY4 = dataclasses.replace(synth.TINY, L=4)


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _bf16_bits(t):
    return t.contiguous().view(dtype=__import__("torch").int16).numpy().view(np.uint16)


@pytest.mark.parametrize("absmax", ["f32", "dq8"])
def test_disk_layers_hold_the_oracle_quantisation(q, tmp_path, absmax):
    cfg = TINY4
    path = tmp_path / "store.bin"
    store = q.Store(cfg, absmax=absmax, ram_layers=0, disk_path=path)
    rec = store.record_bytes
    assert os.path.getsize(path) == cfg.L * (-(-rec // 4096) * 4096)
    assert all(q.qls_store_layer_tier(store.h, l) == q.QLS_TIER_DISK for l in range(cfg.L))
    for l in range(cfg.L):
        ws = synth.base_layer(cfg, l)
        na, nm = synth.layer_norms(cfg, l, perturbed=True)
        store.set_layer_fp32(l, ws, na, nm)
    for l in (2, 0, 3, 1):                          # views in any order
        ws = synth.base_layer(cfg, l)
        na, nm = synth.layer_norms(cfg, l, perturbed=True)
        v = store.layer(l)
        for m, w in enumerate(ws):
            codes, am = nf4.quantize(w)
            assert np.array_equal(v["codes"][m], codes), (l, m)
            if absmax == "f32":
                assert np.array_equal(v["absmax"][m].view(np.uint32), am.view(np.uint32)), (l, m)
            else:
                q8, sc = nf4.double_quant(am)
                assert np.array_equal(v["absmax_q8"][m], q8) and np.array_equal(
                    v["absmax_scale"][m].view(np.uint32), sc.view(np.uint32)), (l, m)
        assert np.array_equal(v["norm_attn"], _bf16_bits(na)) and np.array_equal(v["norm_mlp"], _bf16_bits(nm))
    store.close()
    assert not os.path.exists(path)


def test_tiers_and_errors(q, tmp_path):
    cfg = TINY4
    mc = q.model_cfg(cfg)
    with pytest.raises(q.QlsError) as e:
        q.qls_store_create_tiered(mc, q.QLS_ABSMAX_F32, 5, str(tmp_path / "a.bin"))
    assert e.value.code == q.QLS_EINVAL
    with pytest.raises(q.QlsError) as e:
        q.qls_store_create_tiered(mc, q.QLS_ABSMAX_F32, -1, str(tmp_path / "a.bin"))
    assert e.value.code == q.QLS_EINVAL
    with pytest.raises(q.QlsError) as e:
        q.qls_store_create_tiered(mc, q.QLS_ABSMAX_F32, 0, "")
    assert e.value.code == q.QLS_EINVAL
    with pytest.raises(q.QlsError) as e:
        q.qls_store_create_tiered(mc, q.QLS_ABSMAX_F32, 0, str(tmp_path / "no" / "such" / "dir" / "a.bin"))
    assert e.value.code == q.QLS_EIO
    store = q.Store(cfg, ram_layers=0, disk_path=tmp_path / "b.bin")
    with pytest.raises(q.QlsError) as e:
        store.layer(1)                               # never set
    assert e.value.code == q.QLS_ESTATE
    with pytest.raises(q.QlsError):
        q.qls_store_layer_tier(store.h, 4)
    store.close()
