"""Shared test helpers: build oracle models from the seeded synthetic inputs."""
import numpy as np

import synth
from oracle import model as om

# A very small Llama-style stack for fp64 finite differences.  in = 96 for the
# down projection makes NF4 blocks straddle rows.
MICRO = synth.ModelCfg(L=2, d=64, H=4, KV=2, hd=16, I=96, V=128, eps=1e-5,
                       theta=500000.0, r=4, alpha=8.0)


def bf16_np(t):
    return t.float().numpy()


def oracle_model(cfg, perturbed=True):
    layers = []
    for l in range(cfg.L):
        ws = synth.base_layer(cfg, l)
        na, nm = synth.layer_norms(cfg, l, perturbed)
        layers.append(om.dequant_layer(cfg, ws, bf16_np(na), bf16_np(nm)))
    return om.Model(cfg, layers, bf16_np(synth.embedding(cfg)), bf16_np(synth.lm_head(cfg)),
                    bf16_np(synth.final_norm(cfg, perturbed)))


def rel_l2(a, b):
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def cosine(a, b):
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    return float(a @ b / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))
