"""Seeded synthetic inputs for the streamed QLoRA step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, no rounding rules, no model math).  Both
the CPU oracle (``oracle/``) and the GPU path's tests and benchmark take their
inputs from here, so the two sides see identical bits.

Shapes follow a Llama-style decoder as described on the page "Fine tune an 8B
model on a 4GB laptop GPU (Soup setup)" (section "Step 2, train": 32 decoder
layers) and the resident embedding / LM head arithmetic of section "The number,
and exactly what it means" (vocabulary 128256 x hidden 4096 in bf16 = 2.10 GB).

Distributions:
  * base weights  W[l,m] ~ N(0, 0.02) float32, generator seed 1000 + 10*l + m
  * embedding / LM head ~ N(0, 0.02), stored bf16, drawn in chunks of 8192
    rows with seeds 11*100000 + c / 12*100000 + c
  * RMSNorm weights: ones (or 1 + N(0, 0.1) when ``perturbed``), bf16
  * LoRA A ~ U(-1/sqrt(in), 1/sqrt(in)) (nn.Linear's Kaiming-uniform default),
    seed 2000 + 10*l + m; LoRA B ~ N(0, b_std), seed 2500 + 10*l + m (B = 0 when
    b_std == 0)
  * token ids uniform over the vocabulary
bf16 values are produced by torch's float32 -> bfloat16 cast.
"""
from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass, asdict

import numpy as np
import torch

MODULES = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class ModelCfg:
    L: int        # decoder layers
    d: int        # hidden size
    H: int        # query heads
    KV: int       # key/value heads
    hd: int       # head dim
    I: int        # SwiGLU intermediate size
    V: int        # vocabulary
    eps: float    # RMSNorm epsilon
    theta: float  # RoPE base
    r: int        # LoRA rank
    alpha: float  # LoRA alpha

    def as_dict(self):
        return asdict(self)

    def module_shapes(self):
        """(name, out, in) of the seven adapted linears, in packing order."""
        d, qd, kvd, I = self.d, self.H * self.hd, self.KV * self.hd, self.I
        return [("q", qd, d), ("k", kvd, d), ("v", kvd, d), ("o", d, qd),
                ("gate", I, d), ("up", I, d), ("down", d, I)]


# Tiny Llama-style stack used for fast parity runs.
TINY = ModelCfg(L=2, d=256, H=4, KV=2, hd=64, I=688, V=1024, eps=1e-5,
                theta=500000.0, r=8, alpha=16.0)
# Llama-3.1-8B-shaped stack.
LLAMA8B = ModelCfg(L=32, d=4096, H=32, KV=8, hd=128, I=14336, V=128256,
                   eps=1e-5, theta=500000.0, r=64, alpha=16.0)


def scaled(cfg: ModelCfg, **kw) -> ModelCfg:
    d = cfg.as_dict()
    d.update(kw)
    return ModelCfg(**d)


# ---------------------------------------------------------------- bf16 helpers
def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 samples -> torch bfloat16 tensor (torch's RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def normal(seed: int, shape, std: float, dtype=np.float32) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape, dtype=dtype) * dtype(std)


# ---------------------------------------------------------------- weights
def base_weight(cfg: ModelCfg, layer: int, m: int, std: float = 0.02) -> np.ndarray:
    """float32 [out, in] frozen base weight of module index m of a layer."""
    _, out, inn = cfg.module_shapes()[m]
    return normal(1000 + 10 * layer + m, (out, inn), std)


def base_layer(cfg: ModelCfg, layer: int, threads: int = 1):
    """The seven float32 base weights of one layer (optionally drawn on threads)."""
    if threads <= 1:
        return [base_weight(cfg, layer, m) for m in range(7)]
    with _cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda m: base_weight(cfg, layer, m), range(7)))


def layer_norms(cfg: ModelCfg, layer: int, perturbed: bool = False):
    """(attn_norm, mlp_norm) bf16 [d] each."""
    if not perturbed:
        one = torch.ones(cfg.d, dtype=torch.bfloat16)
        return one, one.clone()
    a = 1.0 + normal(3000 + 2 * layer, (cfg.d,), 0.1)
    b = 1.0 + normal(3001 + 2 * layer, (cfg.d,), 0.1)
    return to_bf16(a), to_bf16(b)


def final_norm(cfg: ModelCfg, perturbed: bool = False) -> torch.Tensor:
    if not perturbed:
        return torch.ones(cfg.d, dtype=torch.bfloat16)
    return to_bf16(1.0 + normal(3999, (cfg.d,), 0.1))


_VOCAB_CHUNK = 8192


def _vocab_matrix(seed: int, cfg: ModelCfg, std: float, threads: int) -> torch.Tensor:
    """[V, d] ~ N(0, std) drawn in row chunks of 8192, chunk c from seed*100000 + c."""
    out = torch.empty(cfg.V, cfg.d, dtype=torch.bfloat16)

    def fill(c):
        r0 = c * _VOCAB_CHUNK
        r1 = min(cfg.V, r0 + _VOCAB_CHUNK)
        out[r0:r1] = to_bf16(normal(seed * 100000 + c, (r1 - r0, cfg.d), std))

    n = (cfg.V + _VOCAB_CHUNK - 1) // _VOCAB_CHUNK
    if threads <= 1:
        for c in range(n):
            fill(c)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n)))
    return out


def embedding(cfg: ModelCfg, std: float = 0.02, threads: int = 1) -> torch.Tensor:
    return _vocab_matrix(11, cfg, std, threads)


def lm_head(cfg: ModelCfg, std: float = 0.02, threads: int = 1) -> torch.Tensor:
    return _vocab_matrix(12, cfg, std, threads)


# ---------------------------------------------------------------- LoRA
def lora_init(cfg: ModelCfg, b_std: float = 1e-3, a_seed: int = 2000,
              b_seed: int = 2500):
    """[layer][module] -> (A float32 [r,in], B float32 [out,r])."""
    out = []
    for l in range(cfg.L):
        mods = {}
        for m, (name, o, i) in enumerate(cfg.module_shapes()):
            bound = 1.0 / np.sqrt(i)
            A = np.random.default_rng(a_seed + 10 * l + m).uniform(
                -bound, bound, (cfg.r, i)).astype(np.float32)
            if b_std == 0.0:
                B = np.zeros((o, cfg.r), np.float32)
            else:
                B = normal(b_seed + 10 * l + m, (o, cfg.r), b_std)
            mods[name] = (A, B)
        out.append(mods)
    return out


def lora_numel(cfg: ModelCfg) -> int:
    return cfg.L * sum(cfg.r * (i + o) for _, o, i in cfg.module_shapes())


def pack_lora(cfg: ModelCfg, lora) -> np.ndarray:
    """Flat float32 vector: layer-major, module order q,k,v,o,gate,up,down,
    each A [r,in] row-major followed by B [out,r] row-major."""
    parts = []
    for l in range(cfg.L):
        for name, _, _ in cfg.module_shapes():
            A, B = lora[l][name]
            parts.append(np.asarray(A, np.float32).reshape(-1))
            parts.append(np.asarray(B, np.float32).reshape(-1))
    return np.concatenate(parts)


def unpack_lora(cfg: ModelCfg, flat) -> list:
    flat = np.asarray(flat)
    out, off = [], 0
    for l in range(cfg.L):
        mods = {}
        for name, o, i in cfg.module_shapes():
            A = flat[off:off + cfg.r * i].reshape(cfg.r, i)
            off += cfg.r * i
            B = flat[off:off + o * cfg.r].reshape(o, cfg.r)
            off += o * cfg.r
            mods[name] = (A, B)
        out.append(mods)
    assert off == flat.size
    return out


# ---------------------------------------------------------------- activations
def token_ids(cfg: ModelCfg, B: int, S: int, seed: int = 7) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, cfg.V, (B, S)).astype(np.int32)


def dpo_pair(cfg: ModelCfg, S: int, prompt_len: int, seeds=(51, 52, 53)):
    """(chosen, rejected) int32 [S] sharing ids[:prompt_len]."""
    prompt = np.random.default_rng(seeds[0]).integers(0, cfg.V, prompt_len)
    c = np.random.default_rng(seeds[1]).integers(0, cfg.V, S - prompt_len)
    r = np.random.default_rng(seeds[2]).integers(0, cfg.V, S - prompt_len)
    return (np.concatenate([prompt, c]).astype(np.int32),
            np.concatenate([prompt, r]).astype(np.int32))


def activation(seed: int, shape, std: float = 1.0) -> torch.Tensor:
    """bf16 activation / upstream-gradient tensor ~ N(0, std)."""
    return to_bf16(normal(seed, shape, std))
