"""One decoder layer of a real step through the CPU oracle, in worker processes.

The per-layer gradient check runs each layer's forward and hand-derived
backward in the oracle (mirror precision), given the state the step handed
that layer: its input checkpoint x_l and the float32 residual gradient
dL/dx_{l+1} arriving from above.  The oracle quantises the layer's seeded
base weights itself; only those two boundary tensors come from the step.
Workers are spawned processes, so many layers run at once.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np


def _init(threads: int):
    from threadpoolctl import threadpool_limits
    threadpool_limits(threads)


def layer_job(job):
    """job: (cfg, layer, x [T, d] float32 (bf16 values), g_out [T, d] float32,
    lora_l {name: (A, B)}, B, S, absmax "f32" | "dq8", perturbed norms).
    Returns (layer, out [T, d], g_in [T, d], {name: (dA, dB)})."""
    import synth
    from oracle import model as om

    cfg, l, x, g_out, lora_l, B, S, absmax, perturbed = job
    P = om.Prec("mirror")
    ws = synth.base_layer(cfg, l)
    na, nm = synth.layer_norms(cfg, l, perturbed)
    lw = om.dequant_layer(cfg, ws, na.float().numpy(), nm.float().numpy(), absmax)
    del ws
    tabs = om.rope_tables(P, S, cfg.hd, cfg.theta)
    out, cache = om.layer_forward(cfg, P, x, lw, lora_l, B, S, tabs)
    g_in, grads = om.layer_backward(cfg, P, cache, g_out, lw, lora_l, B, S, tabs)
    return l, out, np.asarray(g_in, np.float32), grads


def run_layers(jobs, workers: int, threads: int):
    """Runs layer_job over jobs in `workers` spawned processes of `threads`
    BLAS threads each; returns {layer: (out, g_in, grads)}."""
    ctx = mp.get_context("spawn")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    old = os.environ.get("PYTHONPATH")
    os.environ["PYTHONPATH"] = root + (os.pathsep + old if old else "")
    try:
        with ctx.Pool(workers, initializer=_init, initargs=(threads,)) as pool:
            res = pool.map(layer_job, jobs, chunksize=1)
    finally:
        if old is None:
            os.environ.pop("PYTHONPATH", None)
        else:
            os.environ["PYTHONPATH"] = old
    return {l: (out, g_in, grads) for l, out, g_in, grads in res}


def cpu_share(default: int = 16) -> int:
    """Host threads this process may use (the affinity mask), capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(default, n))
