"""GPU parity of causal grouped-query attention (forward and backward) against
the oracle, through the C ABI (qls_attention_fwd / qls_attention_bwd).

Shapes cover head dims 64 and 128, 1 to 8 query heads per kv head (5 too),
one and two sequences, lengths that are not multiples of the 32-row and
64-key blocks, one length that spans many blocks, and the 8B shape at 4096
tokens (32 query heads, 8 kv heads).  Floating outputs are
held to the bar of the step: relative L2 <= 1e-2 and cosine >= 0.999 (the two
sides round the probabilities to bf16 against different running maxima and
sum in different orders), and element by element to 1e-2 rms + 2e-2 |ref| on
99.9% of elements and 10 times that on every element; the log-sum-exp to 1e-5
relative."""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from tests.gpu_util import elementwise, f32, report

pytestmark = pytest.mark.gpu
PM = om.Prec("mirror")

# The last shape is the 8B model's attention at 4096 tokens, the launch the
# seq-4096 step times.
SHAPES = [(1, 64, 4, 2, 64), (2, 200, 8, 2, 128), (1, 300, 5, 1, 128), (1, 257, 8, 8, 64),
          (1, 97, 16, 2, 64), (1, 1024, 8, 2, 128), (1, 4096, 32, 8, 128)]


@pytest.fixture(scope="module")
def q():
    import layer_streamed_qlora_block_amd as q
    return q


def _bf(t):
    return t.float().numpy()


@pytest.mark.parametrize("B,S,H,KV,hd", SHAPES)
def test_attention_matches_oracle(q, B, S, H, KV, hd):
    print(f"attention B={B} S={S} H={H} KV={KV} hd={hd}", flush=True)
    T = B * S
    qkv = synth.activation(100 + S + H, (T, (H + 2 * KV) * hd))
    dout = synth.activation(200 + S + H, (T, H * hd))
    out = torch.empty(T, H * hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, S, dtype=torch.float32, device="cuda")
    dq = torch.empty(T, H * hd, dtype=torch.float32, device="cuda")
    dk = torch.empty(T, KV * hd, dtype=torch.float32, device="cuda")
    dv = torch.empty(T, KV * hd, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qls_attention_ws_bytes(B, S, H, hd), dtype=torch.uint8, device="cuda")
    d_qkv, d_dout = qkv.cuda(), dout.cuda()
    q.qls_attention_fwd(d_qkv, B, S, H, KV, hd, out, lse)
    q.qls_attention_bwd(d_qkv, out, d_dout, lse, B, S, H, KV, hd, dq, dk, dv, ws)
    torch.cuda.synchronize()

    x = _bf(qkv)
    qq = x[:, :H * hd].reshape(T, H, hd)
    kk = x[:, H * hd:(H + KV) * hd].reshape(T, KV, hd)
    vv = x[:, (H + KV) * hd:].reshape(T, KV, hd)
    o, l = om.attention(PM, qq, kk, vv, B, S)
    rr, cc = report("attention out", f32(out).reshape(T, H, hd), o)
    assert rr <= 1e-2 and cc >= 0.999
    elementwise("attention out", f32(out).reshape(T, H, hd), o, 1e-2, 2e-2)
    assert np.allclose(f32(lse), l, rtol=1e-5, atol=1e-5)
    # backward from the GPU's own forward output and LSE, as the step uses them
    og = f32(out).reshape(T, H, hd)
    odq, odk, odv = om.attention_bwd(PM, qq, kk, vv, og, _bf(dout).reshape(T, H, hd), f32(lse), B, S)
    for name, got, want in (("dq", dq, odq), ("dk", dk, odk), ("dv", dv, odv)):
        rr, cc = report(f"attention {name}", f32(got).reshape(want.shape), want)
        assert rr <= 1e-2 and cc >= 0.999, name
        elementwise(f"attention {name}", f32(got).reshape(want.shape), want, 1e-2, 2e-2)


def test_attention_refuses_unsupported_shapes(q):
    buf = torch.empty(1024, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(64, dtype=torch.float32, device="cuda")
    for args in [(1, 8, 4, 2, 96), (1, 8, 6, 4, 64), (1, 8, 18, 2, 64), (0, 8, 4, 2, 64)]:
        with pytest.raises(q.QlsError):
            q.qls_attention_fwd(buf, *args, buf, lse)
