#!/usr/bin/env python3
"""Write tests/golden/sft_8b_seq512.json: the CPU oracle's full 8B-shaped SFT
step (32 layers, batch 1 x seq 512, mirror precision) on the seeded synthetic
inputs -- loss, every LoRA matrix's gradient L2 norm, and 24 sampled entries
of every dA / dB.

Calls only ``oracle/`` and the seeded input module ``synth`` (no GPU code).
The NF4 store is built by the oracle's own quantiser (in worker processes);
dequantised layers are produced on demand so the script stays within ~12 GB.
Run time: ~20 min on 8 cores.

    python tests/golden/make_golden_8b.py [--prec fp64 --out PATH]
"""
import argparse
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402
from oracle import model as om  # noqa: E402
from oracle import nf4  # noqa: E402

CFG = synth.LLAMA8B
S = 512
SAMPLES = 24


def quantize_layer(l):
    ws = synth.base_layer(CFG, l)
    return l, [nf4.quantize(w) for w in ws]


class LazyLayers:
    """model.layers stand-in: dequantises layer l when it is read."""

    def __init__(self, store):
        self.store = store
        self.shapes = [(o, i) for _, o, i in CFG.module_shapes()]
        self.ones = np.ones(CFG.d, np.float32)

    def __len__(self):
        return CFG.L

    def __getitem__(self, l):
        W = {n: nf4.dequant(c, a, sh) for n, (c, a), sh in zip(om.NAMES, self.store[l], self.shapes)}
        return {"W": W, "norm_attn": self.ones, "norm_mlp": self.ones}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--prec", choices=["mirror", "fp64"], default="mirror")
    ap.add_argument("--out", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "sft_8b_seq512.json"))
    args = ap.parse_args()
    t0 = time.time()
    with mp.get_context("spawn").Pool(min(4, os.cpu_count() or 1)) as pool:
        store = dict(pool.imap_unordered(quantize_layer, range(CFG.L)))
    print(f"quantised {CFG.L} layers in {time.time() - t0:.0f} s", flush=True)
    model = om.Model(CFG, LazyLayers(store), synth.embedding(CFG, threads=8).float().numpy(),
                     synth.lm_head(CFG, threads=8).float().numpy(), np.ones(CFG.d, np.float32))
    lora = synth.lora_init(CFG)
    ids = synth.token_ids(CFG, 1, S, seed=41)
    t1 = time.time()
    loss, grads, _ = om.sft_step(CFG, om.Prec(args.prec), model, lora, ids)
    print(f"sft step in {time.time() - t1:.0f} s, loss {loss:.7f}", flush=True)
    rng = np.random.default_rng(99)
    samples, norms = [], []
    for l in range(CFG.L):
        for m, n in enumerate(om.NAMES):
            for w in range(2):
                g = np.asarray(grads[l][n][w], np.float32).reshape(-1)
                norms.append([l, m, w, float(np.linalg.norm(g.astype(np.float64)))])
                for i in rng.integers(0, g.size, SAMPLES):
                    samples.append([l, m, w, int(i), float(g[i])])
    out = {
        "what": f"oracle SFT step, 8B-shaped stack, batch 1 x seq 512, {args.prec} precision",
        "config": CFG.as_dict(), "seq": S, "ids_seed": 41, "lora_b_std": 1e-3,
        "loss": loss, "grad_norms": norms, "samples": samples,
        "made_by": "tests/golden/make_golden_8b.py (oracle only)",
    }
    path = args.out
    with open(path, "w") as f:
        json.dump(out, f)
    print(f"wrote {path} ({len(samples)} samples) in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
