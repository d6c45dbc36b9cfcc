#!/usr/bin/env python3
"""Write golden values of the CPU oracle's full 8B-shaped steps (32 layers) on
the seeded synthetic inputs.

Tasks (file written by default in this folder):
  --task sft --seq 512            sft_8b_seq512.json (mirror) / sft_8b_seq512_fp64.json (--prec fp64):
                                  loss, every LoRA matrix's gradient L2 norm and 24 sampled
                                  entries of every dA / dB; token ids seed 41
  --task sft --seq 4096 --loss-only
                                  sft_8b_seq4096.json: the loss alone (forward sweep and head);
                                  token ids seed 42
  --task dpo --seq 512            dpo_8b_seq512.json: sigmoid DPO (beta 0.1) on one (chosen,
                                  rejected) pair sharing a 128-token prompt (synth.dpo_pair):
                                  loss, pi_c, pi_r, rho_c, rho_r, z, gradient norms and samples

Calls only ``oracle/`` and the seeded input module ``synth`` (no GPU code).
The NF4 store is built by the oracle's own quantiser (in worker processes);
dequantised layers are produced on demand so the script stays within ~12 GB
(~20 GB for the seq-4096 head).  Run time on 8 cores: ~20 min (sft 512),
~40 min (dpo), ~30 min (sft 4096 loss only).

    python tests/golden/make_golden_8b.py [--task sft|dpo] [--seq N] [--loss-only]
                                          [--prec mirror|fp64] [--out PATH]
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
SAMPLES = 24
IDS_SEED = {512: 41, 4096: 42}
DPO_PROMPT, DPO_BETA = 128, 0.1


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


def grad_summary(grads):
    rng = np.random.default_rng(99)
    samples, norms = [], []
    for l in range(CFG.L):
        for m, n in enumerate(om.NAMES):
            for w in range(2):
                g = np.asarray(grads[l][n][w], np.float32).reshape(-1)
                norms.append([l, m, w, float(np.linalg.norm(g.astype(np.float64)))])
                for i in rng.integers(0, g.size, SAMPLES):
                    samples.append([l, m, w, int(i), float(g[i])])
    return norms, samples


def default_out(task, seq, prec):
    tail = "" if prec == "mirror" else "_" + prec
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), f"{task}_8b_seq{seq}{tail}.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--task", choices=["sft", "dpo"], default="sft")
    ap.add_argument("--seq", type=int, default=512)
    ap.add_argument("--loss-only", action="store_true")
    ap.add_argument("--prec", choices=["mirror", "fp64"], default="mirror")
    ap.add_argument("--workers", type=int, default=4)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    path = args.out or default_out(args.task, args.seq, args.prec)
    t0 = time.time()
    with mp.get_context("spawn").Pool(min(args.workers, os.cpu_count() or 1)) as pool:
        store = dict(pool.imap_unordered(quantize_layer, range(CFG.L)))
    print(f"quantised {CFG.L} layers in {time.time() - t0:.0f} s", flush=True)
    model = om.Model(CFG, LazyLayers(store), synth.embedding(CFG, threads=8).float().numpy(),
                     synth.lm_head(CFG, threads=8).float().numpy(), np.ones(CFG.d, np.float32))
    lora = synth.lora_init(CFG)
    P = om.Prec(args.prec)
    t1 = time.time()
    out = {"config": CFG.as_dict(), "seq": args.seq, "lora_b_std": 1e-3,
           "made_by": "tests/golden/make_golden_8b.py (oracle only)"}
    if args.task == "sft":
        ids = synth.token_ids(CFG, 1, args.seq, seed=IDS_SEED[args.seq])
        out["ids_seed"] = IDS_SEED[args.seq]
        out["what"] = (f"oracle SFT step, 8B-shaped stack, batch 1 x seq {args.seq}, {args.prec} precision"
                       + (", loss only" if args.loss_only else ""))
        if args.loss_only:
            out["loss"] = om.sft_loss(CFG, P, model, lora, ids)
        else:
            loss, grads, _ = om.sft_step(CFG, P, model, lora, ids)
            out["loss"] = loss
            out["grad_norms"], out["samples"] = grad_summary(grads)
    else:
        c, r = synth.dpo_pair(CFG, args.seq, DPO_PROMPT)
        out["what"] = (f"oracle DPO step (sigmoid, beta {DPO_BETA}), 8B-shaped stack, chosen and rejected "
                       f"1 x {args.seq} sharing a {DPO_PROMPT}-token prompt, {args.prec} precision")
        out["prompt_len"], out["beta"], out["pair_seeds"] = DPO_PROMPT, DPO_BETA, [51, 52, 53]
        loss, grads, aux = om.dpo_step(CFG, P, model, lora, c, r, DPO_PROMPT, DPO_BETA)
        out["loss"] = loss
        out["pi"] = [float(x) for x in aux["pi"]]
        out["ref"] = [float(x) for x in aux["ref"]]
        out["z"] = float(aux["z"])
        out["grad_norms"], out["samples"] = grad_summary(grads)
    print(f"{args.task} step in {time.time() - t1:.0f} s, loss {out['loss']:.7f}", flush=True)
    with open(path, "w") as f:
        json.dump(out, f)
    print(f"wrote {path} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
