"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-side pieces (codebook, quantiser, sizes, error
paths) agree with the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def test_exports_every_declared_symbol(q):
    hdr = open(os.path.join(ROOT, "include", "qls.h")).read()
    declared = set(re.findall(r"\b(qls_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 25
    lib = ctypes.CDLL(q.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(q.exported_symbols())
    assert q.qls_abi_version() == 3


def test_codebook_bitwise_equals_oracle(q):
    ours = q.qls_nf4_codebook()
    assert np.array_equal(ours.view(np.uint32), nf4.codebook().view(np.uint32))


@pytest.mark.parametrize("shape,seed", [((256, 688), 1), ((64, 4096), 2), ((14336 // 56, 4096), 3)])
def test_quantizer_bitwise_equals_oracle(q, shape, seed):
    w = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(0.02)
    c1, a1 = q.qls_nf4_quantize(w, n_threads=4)
    c2, a2 = nf4.quantize(w)
    assert np.array_equal(a1.view(np.uint32), a2.view(np.uint32))
    assert np.array_equal(c1, c2)


def test_quantizer_edge_blocks(q):
    cb = nf4.codebook()
    w = np.random.default_rng(4).standard_normal(64 * 6).astype(np.float32)
    w[64:128] = 0.0                                      # all-zero block
    w[128:192] = -0.0                                    # negative zeros
    w[192] = -5.0                                        # absmax on a negative element
    blk = w[256:320]                                     # exact midpoints between levels (ties)
    blk[0] = 1.0
    for j in range(1, 15):
        blk[j] = np.float32((np.float64(cb[j]) + np.float64(cb[j + 1])) / 2)
    w[320:384] = np.float32(1e-30) * np.arange(64, dtype=np.float32)   # tiny values
    c1, a1 = q.qls_nf4_quantize(w, n_threads=1)
    c2, a2 = nf4.quantize(w)
    assert np.array_equal(c1, c2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))


def test_sizes_match_the_8b_arithmetic(q):
    mc = q.model_cfg(synth.LLAMA8B)
    # codes 109,051,904 + absmax 13,631,488 + two 4096-wide bf16 norms
    assert q.qls_layer_record_bytes(mc) == 122_699_776
    assert q.qls_lora_numel(mc) == 167_772_160 == synth.lora_numel(synth.LLAMA8B)
    assert q.qls_lora_numel(q.model_cfg(synth.TINY)) == synth.lora_numel(synth.TINY)


def test_error_paths(q):
    with pytest.raises(q.QlsError) as e:
        q.qls_nf4_quantize(np.zeros(65, np.float32))
    assert e.value.code == q.QLS_EINVAL
    bad = q.model_cfg(synth.scaled(synth.TINY, KV=3))
    with pytest.raises(q.QlsError) as e:
        q.qls_layer_record_bytes(bad)
    assert e.value.code == q.QLS_EINVAL and "multiple" in q.last_error()
    with pytest.raises(q.QlsError) as e:                 # cap smaller than the store
        q.qls_store_create(q.model_cfg(synth.TINY), max_pinned_bytes=1024)
    assert e.value.code == q.QLS_ENOPIN
    q.qls_store_destroy(None)                            # NULL-safe
    q.qls_session_destroy(None)
    with pytest.raises(q.QlsError):
        q.qls_linear_ws_bytes(0, 16, 16, 8)


@pytest.mark.parametrize("nb,seed", [(256, 1), (1000, 2), (3, 3), (4096 * 7 + 5, 4)])
def test_double_quant_bitwise_equals_oracle(q, nb, seed):
    rng = np.random.default_rng(seed)
    a = np.abs(rng.normal(0, 0.02, (nb, 64))).max(axis=1).astype(np.float32)
    a[: min(nb, 17)] *= np.float32(3.0)            # a few large entries per group
    if nb > 600:
        a[256:512] = 0                            # an all-zero group
    q8, s = q.qls_nf4_double_quant(a)
    q8o, so = nf4.double_quant(a)
    assert np.array_equal(q8, q8o) and np.array_equal(s.view(np.uint32), so.view(np.uint32))


def test_double_quant_record_size(q):
    mc = q.model_cfg(synth.LLAMA8B)
    # codes 109,051,904 + 8-bit absmax 3,407,872 + 13,312 group scales + norms
    assert q.qls_layer_record_bytes_fmt(mc, q.QLS_ABSMAX_DQ8) == 112_529_408
    assert q.qls_layer_record_bytes_fmt(mc, q.QLS_ABSMAX_F32) == q.qls_layer_record_bytes(mc)
    with pytest.raises(q.QlsError) as e:
        q.qls_layer_record_bytes_fmt(mc, 7)
    assert e.value.code == q.QLS_EINVAL
