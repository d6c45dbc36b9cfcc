"""The allocation-free attention backward (qls_attention_bwd_noalloc) against
qls_attention_bwd, through the C ABI: the same kernels over a fixed device
scratch array instead of a caller workspace, so dq, dk and dv must equal the
workspace entry point's bit for bit.  Two calls in a row, the second smaller
(its scratch still holds the first call's contents), then the first shape
again; a problem larger than the fixed scratch is refused before any launch.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _problem(q, B, S, H, KV, hd, seed):
    T = B * S
    qkv = synth.activation(seed, (T, (H + 2 * KV) * hd)).cuda()
    dout = synth.activation(seed + 1, (T, H * hd)).cuda()
    out = torch.empty(T, H * hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, S, dtype=torch.float32, device="cuda")
    q.qls_attention_fwd(qkv, B, S, H, KV, hd, out, lse)
    return qkv, dout, out, lse


def _grads(T, H, KV, hd):
    return (torch.full((T, H * hd), float("nan"), device="cuda"),
            torch.full((T, KV * hd), float("nan"), device="cuda"),
            torch.full((T, KV * hd), float("nan"), device="cuda"))


def _with_workspace(q, prob, B, S, H, KV, hd):
    qkv, dout, out, lse = prob
    dq, dk, dv = _grads(B * S, H, KV, hd)
    ws = torch.empty(q.qls_attention_ws_bytes(B, S, H, hd), dtype=torch.uint8, device="cuda")
    q.qls_attention_bwd(qkv, out, dout, lse, B, S, H, KV, hd, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return [bits(t) for t in (dq, dk, dv)]


def _no_alloc(q, prob, B, S, H, KV, hd):
    qkv, dout, out, lse = prob
    dq, dk, dv = _grads(B * S, H, KV, hd)
    q.qls_attention_bwd_noalloc(qkv, out, dout, lse, B, S, H, KV, hd, dq, dk, dv)
    torch.cuda.synchronize()
    return [bits(t) for t in (dq, dk, dv)]


# The 8B attention shape at 1024 tokens (33.7 MB of scratch: near the 40 MiB
# limit), then a smaller, ragged problem with hd 64 and two sequences.
BIG = (1, 1024, 32, 8, 128)
SMALL = (2, 200, 8, 2, 64)


def test_no_alloc_attention_bwd_equals_workspace_entry_point(q):
    probs = {BIG: _problem(q, *BIG, seed=401), SMALL: _problem(q, *SMALL, seed=402)}
    want = {shape: _with_workspace(q, probs[shape], *shape) for shape in (BIG, SMALL)}
    for shape in (BIG, SMALL, BIG):
        print(f"no-alloc attention backward B,S,H,KV,hd = {shape}", flush=True)
        got = _no_alloc(q, probs[shape], *shape)
        for name, g, w in zip(("dq", "dk", "dv"), got, want[shape]):
            assert np.array_equal(g, w), (shape, name)
            assert np.all(np.isfinite(g.view(np.float32))), (shape, name)


def test_no_alloc_refuses_problems_beyond_its_scratch(q):
    B, S, H, KV, hd = 1, 1276, 32, 8, 128          # 41.98 MB > 40 MiB
    assert q.qls_attention_ws_bytes(B, S, H, hd) > q.QLS_NOALLOC_SCRATCH_BYTES
    buf = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    f = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QlsError) as e:
        q.qls_attention_bwd_noalloc(buf, buf, buf, f, B, S, H, KV, hd, f, f, f)
    assert e.value.code == q.QLS_EINVAL
    # the entry point still works afterwards
    prob = _problem(q, *SMALL, seed=403)
    assert all(np.array_equal(a, b) for a, b in zip(_no_alloc(q, prob, *SMALL), _with_workspace(q, prob, *SMALL)))
