"""Decoder stack, hand-derived LoRA backward, cross-entropy and DPO -- oracle side.

Test infrastructure only (see ``oracle/__init__``).  Plain NumPy, one code
path, two precision modes:

  ``fp64``    float64 everywhere, no rounding (finite differences).
  ``mirror``  float32 math with bf16 round-to-nearest-even applied exactly at
              the storage points listed below (the precision contract that the
              GPU path also follows).

What is computed (the un-streamed step; streaming is a reordering only, page
"Soup ... radar note", section "In detail"):
  * LoRA on a frozen base: only the adapter matrices receive gradients (page
    "Can You Fine-Tune Llama 3.1 8B on a 4GB GPU? ...", section "How Soup's
    layer streaming actually works", item 1).
  * Gradient checkpointing: only the layer inputs are kept; each layer's
    forward is recomputed when its backward runs (same page and section,
    item 4).
  * Embedding and LM head resident, logits over the vocabulary (page "Fine tune
    an 8B model ... (Soup setup)", section "The number, and exactly what it
    means").
  * DPO reference = the same base with the adapters disabled (page "Soup ...
    radar note", section "In detail").

Precision contract (mirror mode):
  PC1  weight operand = NF4 dequant: bf16(float32(cb[c] * absmax)).
  PC2  GEMM operands bf16, float32 accumulation, one rounding on store.
  PC3  LoRA masters float32, bf16 copies are the GEMM operands; u = x A^T is
       stored bf16; base + s * (u B^T) + residual summed in float32, one
       rounding.
  PC4  RMSNorm / softmax / CE statistics in float32.
  PC5  activations between ops bf16.
  PC6  residual-gradient stream float32 across layers; dY GEMM operands bf16.
  PC7  dA, dB accumulated and returned in float32.
  PC8  attention probabilities rounded to bf16 as the operand of P V and of
       P^T dO.
  PC9  loss terms float32, summed in float64.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import nf4

NAMES = ("q", "k", "v", "o", "gate", "up", "down")


class Prec:
    """Precision mode: ``fp64`` (no rounding) or ``mirror`` (float32 + bf16 rounding)."""

    def __init__(self, mode: str = "mirror"):
        if mode not in ("mirror", "fp64"):
            raise ValueError(mode)
        self.mode = mode
        self.dt = np.float64 if mode == "fp64" else np.float32

    def c(self, x):
        return np.asarray(x, dtype=self.dt)

    def rb(self, x):
        x = np.asarray(x)
        if self.mode == "fp64":
            return x.astype(np.float64)
        return nf4.bf16_bits_to_f32(nf4.bf16_bits_rne(x.astype(np.float32))).reshape(x.shape)


@dataclass
class Model:
    """Frozen model, every array holding bf16 values (as float32)."""
    cfg: object                 # synth.ModelCfg-like (L, d, H, KV, hd, I, V, eps, theta, r, alpha)
    layers: list                # [{"W": {name: [out,in]}, "norm_attn": [d], "norm_mlp": [d]}]
    embed: np.ndarray           # [V, d]
    lm_head: np.ndarray         # [V, d]
    final_norm: np.ndarray      # [d]


def dequant_layer(cfg, weights_fp32, norm_attn, norm_mlp, absmax="f32"):
    """Quantise the seven float32 weights with the oracle's NF4 and dequantise;
    absmax="dq8" double-quantises each weight's absmax first."""
    W = {}
    for name, w in zip(NAMES, weights_fp32):
        codes, amax = nf4.quantize(w)
        if absmax == "dq8":
            W[name] = nf4.dequant_dq(codes, *nf4.double_quant(amax), w.shape)
        else:
            W[name] = nf4.dequant(codes, amax, w.shape)
    return {"W": W, "norm_attn": np.asarray(norm_attn, np.float32),
            "norm_mlp": np.asarray(norm_mlp, np.float32)}


# ------------------------------------------------------------------ blocks
def rmsnorm(P, x, w, eps):
    """y = x * (mean(x^2) + eps)^-1/2 * w, one rounding; returns (y, rho)."""
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=P.dt)
    rho = (P.c(1.0) / np.sqrt(ms + P.c(eps))).astype(P.dt)
    return P.rb(x * rho * P.c(w)), rho


def rmsnorm_bwd(P, x, w, rho, dy):
    """dx = rho * (dy*w - xhat * mean(dy*w*xhat)), xhat = rho*x."""
    xhat = x * rho
    dyw = dy * P.c(w)
    return rho * (dyw - xhat * np.mean(dyw * xhat, axis=-1, keepdims=True, dtype=P.dt))


def rope_tables(P, S, hd, theta):
    """cos/sin [S, hd/2]; inv_freq_j = theta^(-2j/hd) (float64 then P.dt), angle = pos * inv_freq."""
    j = np.arange(hd // 2, dtype=np.float64)
    inv = (float(theta) ** (-2.0 * j / hd)).astype(P.dt)
    pos = np.arange(S).astype(P.dt)
    ang = (pos[:, None] * inv[None, :]).astype(P.dt)
    a64 = ang.astype(np.float64)
    return np.cos(a64).astype(P.dt), np.sin(a64).astype(P.dt)


def rope(P, x, cos, sin, B, inverse=False):
    """Rotate-half RoPE on x [T, nh, hd]: pairs (j, j + hd/2) rotated by pos*inv_freq_j."""
    h = x.shape[-1] // 2
    c = np.tile(cos, (B, 1))[:, None, :]
    s = np.tile(sin, (B, 1))[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    if not inverse:
        y1, y2 = x1 * c - x2 * s, x2 * c + x1 * s
    else:
        y1, y2 = x1 * c + x2 * s, x2 * c - x1 * s
    return P.rb(np.concatenate([y1, y2], axis=-1))


def attention(P, q, k, v, B, S):
    """Causal GQA attention.  q [T,H,hd], k/v [T,KV,hd] -> o [T,H,hd], lse [B,H,S].

    Head h reads kv head h // (H/KV); scores = q k^T / sqrt(hd) with j <= i;
    o = bf16( bf16(exp(s - max)) v / sum(exp(s - max)) )."""
    T, H, hd = q.shape
    grp = H // k.shape[1]
    scale = P.c(1.0 / np.sqrt(hd))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    o = np.empty((T, H, hd), P.dt)
    lse = np.empty((B, H, S), P.dt)
    for b in range(B):
        sl = slice(b * S, (b + 1) * S)
        for h in range(H):
            g = h // grp
            s = (q[sl, h] @ k[sl, g].T) * scale
            s[mask] = -np.inf
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True, dtype=P.dt)
            o[sl, h] = P.rb((P.rb(p) @ v[sl, g]) / l)
            lse[b, h] = (m + np.log(l))[:, 0]
    return o, lse


def attention_bwd(P, q, k, v, o, do, lse, B, S):
    """dV = P^T dO; dP = dO V^T; dS = P (dP - rowsum(dO o)); dQ = dS K / sqrt(hd);
    dK = dS^T Q / sqrt(hd); dK, dV summed over each query-head group."""
    T, H, hd = q.shape
    KV = k.shape[1]
    grp = H // KV
    scale = P.c(1.0 / np.sqrt(hd))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    dq = np.zeros((T, H, hd), P.dt)
    dk = np.zeros((T, KV, hd), P.dt)
    dv = np.zeros((T, KV, hd), P.dt)
    for b in range(B):
        sl = slice(b * S, (b + 1) * S)
        for h in range(H):
            g = h // grp
            s = (q[sl, h] @ k[sl, g].T) * scale
            s[mask] = -np.inf
            p = np.exp(s - lse[b, h][:, None])
            dv[sl, g] += P.rb(p).T @ do[sl, h]
            dp = do[sl, h] @ v[sl, g].T
            D = np.sum(do[sl, h] * o[sl, h], axis=1, keepdims=True, dtype=P.dt)
            ds = P.rb(p * (dp - D))
            dq[sl, h] = (ds @ k[sl, g]) * scale
            dk[sl, g] += (ds.T @ q[sl, h]) * scale
    return dq, dk, dv


def swiglu(P, g, u):
    with np.errstate(over="ignore"):
        sig = P.c(1.0) / (P.c(1.0) + np.exp(-g))
    return P.rb(g * sig * u)


def swiglu_bwd(P, da, g, u):
    """a = silu(g) u: dg = da u sig (1 + g (1 - sig)); du = da silu(g)."""
    one = P.c(1.0)
    with np.errstate(over="ignore"):
        sig = one / (one + np.exp(-g))
    dg = da * u * sig * (one + g * (one - sig))
    du = da * (g * sig)
    return P.rb(dg), P.rb(du)


def lora_linear(P, x, W, ab, s, residual=None):
    """y = bf16(x W^T + s * u bf16(B)^T [+ residual]), u = bf16(x bf16(A)^T); returns (y, u)."""
    acc = x @ P.c(W).T
    u = None
    if ab is not None:
        A, Bm = ab
        u = P.rb(x @ P.rb(A).T)
        acc = acc + P.c(s) * (u @ P.rb(Bm).T)
    if residual is not None:
        acc = acc + residual
    return P.rb(acc), u


def lora_linear_bwd(P, x, u, W, ab, s, dy):
    """Backward of y = x W^T + s u B^T, u = x A^T, for an upstream dy (bf16 values).

    du = bf16(s dy B);  dA = du^T x;  dB = s dy^T u;  dx = dy W + du A.
    Returns (dx, (dA, dB)) with (dA, dB) None when the adapters are disabled."""
    dx = dy @ P.c(W)
    if ab is None:
        return dx, None
    A, Bm = ab
    s = P.c(s)
    du = P.rb(s * (dy @ P.rb(Bm)))
    return dx + du @ P.rb(A), (du.T @ x, s * (dy.T @ u))


# ------------------------------------------------------------------ layer
def layer_forward(cfg, P, x, lw, lora_l, B, S, tabs):
    """One decoder layer.  x [T, d] (bf16 values) -> (out [T, d], cache)."""
    T = B * S
    H, KV, hd = cfg.H, cfg.KV, cfg.hd
    s = cfg.alpha / cfg.r
    W = lw["W"]
    ab = (lambda n: None) if lora_l is None else (lambda n: lora_l[n])
    c = {"x": x}
    c["n1"], c["rho1"] = rmsnorm(P, x, lw["norm_attn"], cfg.eps)
    q, c["uq"] = lora_linear(P, c["n1"], W["q"], ab("q"), s)
    k, c["uk"] = lora_linear(P, c["n1"], W["k"], ab("k"), s)
    v, c["uv"] = lora_linear(P, c["n1"], W["v"], ab("v"), s)
    cos, sin = tabs
    c["qr"] = rope(P, q.reshape(T, H, hd), cos, sin, B)
    c["kr"] = rope(P, k.reshape(T, KV, hd), cos, sin, B)
    c["v"] = v.reshape(T, KV, hd)
    o, c["lse"] = attention(P, c["qr"], c["kr"], c["v"], B, S)
    c["attn"] = o.reshape(T, H * hd)
    c["h"], c["uo"] = lora_linear(P, c["attn"], W["o"], ab("o"), s, residual=x)
    c["n2"], c["rho2"] = rmsnorm(P, c["h"], lw["norm_mlp"], cfg.eps)
    c["g"], c["ug"] = lora_linear(P, c["n2"], W["gate"], ab("gate"), s)
    c["u"], c["uu"] = lora_linear(P, c["n2"], W["up"], ab("up"), s)
    c["a"] = swiglu(P, c["g"], c["u"])
    out, c["ud"] = lora_linear(P, c["a"], W["down"], ab("down"), s, residual=c["h"])
    return out, c


def layer_backward(cfg, P, c, g_out, lw, lora_l, B, S, tabs):
    """Hand-derived backward of one layer.  g_out [T, d] float (dL/d out).

    LoRA linear y = x W^T + s (x A^T) B^T with u = x A^T:
      dB = s dY^T u,  du = s dY B,  dA = du^T x,  dX = dY W + du A.
    Returns (g_in [T, d], {name: (dA [r,in], dB [out,r])})."""
    T = B * S
    H, KV, hd = cfg.H, cfg.KV, cfg.hd
    s = P.c(cfg.alpha / cfg.r)
    W = lw["W"]
    grads = {}

    def lin_bwd(name, x_in, u, dy):
        dx, g = lora_linear_bwd(P, x_in, u, W[name], None if lora_l is None else lora_l[name], s, dy)
        if g is not None:
            grads[name] = g
        return dx

    dy_down = P.rb(g_out)
    da = lin_bwd("down", c["a"], c["ud"], dy_down)
    dg, du = swiglu_bwd(P, da, c["g"], c["u"])
    dn2 = lin_bwd("gate", c["n2"], c["ug"], dg) + lin_bwd("up", c["n2"], c["uu"], du)
    dh = g_out + rmsnorm_bwd(P, c["h"], lw["norm_mlp"], c["rho2"], dn2)
    dattn = P.rb(lin_bwd("o", c["attn"], c["uo"], P.rb(dh)))
    dqr, dkr, dv = attention_bwd(P, c["qr"], c["kr"], c["v"], c["attn"].reshape(T, H, hd),
                                 dattn.reshape(T, H, hd), c["lse"], B, S)
    cos, sin = tabs
    dq = rope(P, dqr, cos, sin, B, inverse=True).reshape(T, H * hd)
    dk = rope(P, dkr, cos, sin, B, inverse=True).reshape(T, KV * hd)
    dvb = P.rb(dv).reshape(T, KV * hd)
    dn1 = (lin_bwd("q", c["n1"], c["uq"], dq) + lin_bwd("k", c["n1"], c["uk"], dk)
           + lin_bwd("v", c["n1"], c["uv"], dvb))
    g_in = dh + rmsnorm_bwd(P, c["x"], lw["norm_attn"], c["rho1"], dn1)
    return g_in, grads


# ------------------------------------------------------------------ head
def targets(ids):
    """Row t of a sequence predicts ids[t+1]; the last row of each sequence has none (-1)."""
    B, S = ids.shape
    tgt = np.full((B, S), -1, dtype=np.int64)
    tgt[:, :-1] = ids[:, 1:]
    return tgt.reshape(-1)


def head_forward(cfg, P, model, xL):
    """Final RMSNorm, logits = hf W_lm^T (float accumulate), per-row log-sum-exp."""
    hf, rho = rmsnorm(P, xL, model.final_norm, cfg.eps)
    logits = hf @ P.c(model.lm_head).T
    m = logits.max(axis=1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(logits - m), axis=1, keepdims=True, dtype=P.dt)))[:, 0]
    return {"hf": hf, "rho": rho, "logits": logits, "lse": lse.astype(P.dt)}


def row_logp(hc, tgt):
    """log softmax(logits_t)[tgt_t] per row (0 where tgt < 0)."""
    T = tgt.size
    ok = tgt >= 0
    tl = np.zeros(T, hc["logits"].dtype)
    tl[ok] = hc["logits"][np.arange(T)[ok], tgt[ok]]
    return np.where(ok, tl - hc["lse"], 0.0).astype(hc["logits"].dtype)


def head_backward(cfg, P, model, xL, hc, tgt, w_rows):
    """dlogits = w_t (softmax - onehot(tgt_t)); dhf = bf16(dlogits) W_lm; back through the final norm."""
    T = tgt.size
    prob = np.exp(hc["logits"] - hc["lse"][:, None])
    ok = tgt >= 0
    prob[np.arange(T)[ok], tgt[ok]] -= 1.0
    dl = prob * P.c(w_rows)[:, None]
    dhf = P.rb(dl) @ P.c(model.lm_head)
    return rmsnorm_bwd(P, xL, model.final_norm, hc["rho"], dhf)


# ------------------------------------------------------------------ steps
def _embed(P, model, ids):
    return P.c(model.embed[np.asarray(ids).reshape(-1)])


def forward_sweep(cfg, P, model, lora, ids, x0=None):
    """Returns (checkpoints x_0..x_L, tabs)."""
    B, S = ids.shape
    tabs = rope_tables(P, S, cfg.hd, cfg.theta)
    x = _embed(P, model, ids) if x0 is None else P.c(x0)
    xs = [x]
    for l in range(cfg.L):
        x, _ = layer_forward(cfg, P, x, model.layers[l],
                             None if lora is None else lora[l], B, S, tabs)
        xs.append(x)
    return xs, tabs


def backward_sweep(cfg, P, model, lora, xs, g, B, S, tabs):
    """Recompute each layer from its checkpoint, then back-propagate.  Returns (g_0, grads)."""
    grads = [None] * cfg.L
    for l in reversed(range(cfg.L)):
        lora_l = None if lora is None else lora[l]
        _, c = layer_forward(cfg, P, xs[l], model.layers[l], lora_l, B, S, tabs)
        g, grads[l] = layer_backward(cfg, P, c, g, model.layers[l], lora_l, B, S, tabs)
    return g, grads


def _sft_forward(cfg, P, model, lora, ids, x0=None):
    """Forward sweep, head and the mean next-token cross-entropy over the
    B*(S-1) targets.  Returns (loss, xs, tabs, hc, tgt, w)."""
    B, S = ids.shape
    xs, tabs = forward_sweep(cfg, P, model, lora, ids, x0)
    hc = head_forward(cfg, P, model, xs[-1])
    tgt = targets(ids)
    N = B * (S - 1)
    w = np.where(tgt >= 0, 1.0 / N, 0.0)
    terms = -row_logp(hc, tgt)
    loss = float(np.sum(terms.astype(np.float64) * w))
    return loss, xs, tabs, hc, tgt, w


def sft_loss(cfg, P, model, lora, ids):
    """The SFT step's loss alone (forward sweep and head, no backward)."""
    return _sft_forward(cfg, P, model, lora, np.asarray(ids))[0]


def sft_step(cfg, P, model, lora, ids, x0=None):
    """One SFT step: next-token cross-entropy, mean over the B*(S-1) targets.

    Returns (loss, grads[l][name] = (dA, dB), aux) with aux holding the layer
    input checkpoints and g_0 = dL/dx_0."""
    ids = np.asarray(ids)
    B, S = ids.shape
    loss, xs, tabs, hc, tgt, w = _sft_forward(cfg, P, model, lora, ids, x0)
    g = head_backward(cfg, P, model, xs[-1], hc, tgt, w)
    g0, grads = backward_sweep(cfg, P, model, lora, xs, g, B, S, tabs)
    return loss, grads, {"xs": xs, "g0": g0, "lse": hc["lse"], "logits": hc["logits"]}


def seq_logprobs(cfg, P, model, lora, ids, prompt_len):
    """Per sequence: sum over t in [prompt_len, S) of log softmax(logits_{t-1})[ids_t].
    ``lora=None`` disables the adapters (the DPO reference pass)."""
    ids = np.asarray(ids)
    B, S = ids.shape
    xs, _ = forward_sweep(cfg, P, model, lora, ids)
    hc = head_forward(cfg, P, model, xs[-1])
    lp = row_logp(hc, targets(ids)).reshape(B, S)
    return lp[:, prompt_len - 1:S - 1].astype(np.float64).sum(axis=1), lp


def dpo_step(cfg, P, model, lora, chosen, rejected, prompt_len, beta):
    """Sigmoid DPO on one (chosen, rejected) pair against the adapters-disabled reference.

    z = beta((pi_c - rho_c) - (pi_r - rho_r)), L = softplus(-z),
    dL/dpi_c = -beta sigmoid(-z), dL/dpi_r = +beta sigmoid(-z)."""
    ids = np.stack([np.asarray(chosen), np.asarray(rejected)])
    B, S = ids.shape
    ref, _ = seq_logprobs(cfg, P, model, None, ids, prompt_len)
    xs, tabs = forward_sweep(cfg, P, model, lora, ids)
    hc = head_forward(cfg, P, model, xs[-1])
    tgt = targets(ids)
    lp = row_logp(hc, tgt).reshape(B, S)
    pol = lp[:, prompt_len - 1:S - 1].astype(np.float64).sum(axis=1)
    z = beta * ((pol[0] - ref[0]) - (pol[1] - ref[1]))
    loss = float(np.logaddexp(0.0, -z))
    sig = 1.0 / (1.0 + np.exp(z))          # sigmoid(-z)
    dpi = np.array([-beta * sig, beta * sig])
    w = np.zeros((B, S))
    w[:, prompt_len - 1:S - 1] = -dpi[:, None]
    g = head_backward(cfg, P, model, xs[-1], hc, tgt, w.reshape(-1))
    _, grads = backward_sweep(cfg, P, model, lora, xs, g, B, S, tabs)
    return loss, grads, {"pi": pol, "ref": ref, "z": z}


def pref_step(cfg, P, model, lora, chosen, rejected, prompt_len, kind, **params):
    """One preference step of head ``kind`` (oracle.pref) on one (chosen,
    rejected) pair that shares ids[:prompt_len]: the adapters-disabled
    reference pass for the heads that use one, the policy pass, the head on the
    response log-likelihoods, and the backward of -dL/dpi_x spread over each
    response token's log-probability into the LoRA matrices."""
    from . import pref
    ids = np.stack([np.asarray(chosen), np.asarray(rejected)])
    B, S = ids.shape
    n = (S - prompt_len, S - prompt_len)
    ref = (np.zeros(2) if not pref.needs_reference(kind)
           else seq_logprobs(cfg, P, model, None, ids, prompt_len)[0])
    xs, tabs = forward_sweep(cfg, P, model, lora, ids)
    hc = head_forward(cfg, P, model, xs[-1])
    tgt = targets(ids)
    lp = row_logp(hc, tgt).reshape(B, S)
    pol = lp[:, prompt_len - 1:S - 1].astype(np.float64).sum(axis=1)
    loss, dpi = pref.head(kind, pol, ref, n, **params)
    w = np.zeros((B, S))
    w[:, prompt_len - 1:S - 1] = -np.asarray(dpi)[:, None]
    g = head_backward(cfg, P, model, xs[-1], hc, tgt, w.reshape(-1))
    _, grads = backward_sweep(cfg, P, model, lora, xs, g, B, S, tabs)
    return float(loss), grads, {"pi": pol, "ref": np.asarray(ref, dtype=np.float64), "dpi": dpi}
