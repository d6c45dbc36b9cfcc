#!/usr/bin/env python3
"""Benchmark of the streamed QLoRA SFT step on the 8B-shaped stack, one MI355X.

Workload (one step = the whole hot path): 32 Llama-3.1-8B-shaped decoder
layers held as NF4 (block 64; absmax double-quantised by default, ``--absmax
f32`` for float32 absmax) in pinned host memory, streamed one
layer ahead through two device slots; resident bf16 embedding and LM head
(128256 x 4096); LoRA r=64, alpha=16 on the seven linears; batch 1 x seq 512
(``--seq 4096`` for the long-sequence case); forward sweep, vocabulary-chunked
cross-entropy, backward sweep with recomputation, LoRA gradients only.  All
inputs are seeded synthetic tensors of those shapes (``synth``), resident in
device memory before the timed region (the layer store in pinned host memory,
as the method streams it from there).

Prints one JSON line: tokens/s over the timed steps plus the dequant-GEMM
roofline (hipEvents around every launch on the compute stream), the
host-to-device copy rate under overlap against the isolated pinned copy rate,
peak device memory, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "streamed QLoRA SFT tokens/sec (8B-shape, seq 512); % H2D BW and % MFMA peak"
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
# HBM bytes per launch of a dequant-GEMM kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE passes scaled by a known-size copy (profiles/hbm_traffic_dequant_gemm_8b.md);
# valid only for the kernel code they were taken on, keyed by (kernel, sequence length).
TRAFFIC_BYTES_PER_LAUNCH = {("dq_fwd_256", 512): 165.5e6, ("dq_fwd_256", 4096): 755.6e6}
PCIE_GEN5_X16_GBPS = 64.0       # theoretical per direction


def gpu_clock_mhz():
    """Best effort: the current sclk from rocm-smi, run as a child process.  Skipped
    under a profiler, whose preloaded library would initialise the GPU in the
    child before rocm-smi's interpreter starts."""
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return None
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if "sclk" in line and "Mhz" in line:
                return line.split("(")[-1].split("Mhz")[0].strip() + " MHz"
    except Exception:
        pass
    return None


def build_store(q, synth, cfg, threads, absmax, disk_layers=0, disk_dir=None):
    if disk_layers > 0:
        path = os.path.join(disk_dir or os.environ.get("TMPDIR", "/tmp"), f"qls_store_{os.getpid()}.bin")
        store = q.Store(cfg, absmax=absmax, ram_layers=cfg.L - disk_layers, disk_path=path)
    else:
        store = q.Store(cfg, absmax=absmax)
    per = max(1, threads // 4)

    def one(l):
        ws = synth.base_layer(cfg, l, threads=per)
        na, nm = synth.layer_norms(cfg, l)
        store.set_layer_fp32(l, ws, na, nm, n_threads=per)
        return l

    with cf.ThreadPoolExecutor(4) as ex:
        list(ex.map(one, range(cfg.L)))
    return store


def h2d_isolated_gbps(torch, nbytes, iters=20):
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    times = []
    with torch.cuda.stream(s):
        for i in range(iters + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            dst.copy_(src, non_blocking=True)
            b.record(s)
            b.synchronize()
            if i >= 2:
                times.append(a.elapsed_time(b))
    times.sort()
    return nbytes / (times[len(times) // 2] * 1e-3) / 1e9


def cpu_baseline(synth, cfg, T, threads):
    """The oracle, untouched, timed on one decoder layer (NF4 decode + forward +
    recomputed forward + backward) and the LM head (forward + backward) at T
    tokens; the step time is scaled as L * layer + head."""
    import numpy as np
    from oracle import model as om
    from oracle import nf4
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = os.cpu_count()
    one = synth.scaled(cfg, L=1)
    ws = synth.base_layer(one, 0, threads=threads)
    with cf.ThreadPoolExecutor(7) as ex:                 # store build: untimed
        q = list(ex.map(nf4.quantize, ws))
    P = om.Prec("mirror")
    S = T
    x = synth.activation(31, (T, cfg.d)).float().numpy()
    g = synth.activation(32, (T, cfg.d)).float().numpy() * np.float32(1e-3)
    lora = synth.lora_init(one)
    ones = np.ones(cfg.d, np.float32)
    t0 = time.perf_counter()
    W = {n: nf4.dequant(c, a, w.shape) for n, (c, a), w in zip(om.NAMES, q, ws)}
    lw = {"W": W, "norm_attn": ones, "norm_mlp": ones}
    tabs = om.rope_tables(P, S, cfg.hd, cfg.theta)
    om.layer_forward(one, P, x, lw, lora[0], 1, S, tabs)                  # forward sweep
    _, c = om.layer_forward(one, P, x, lw, lora[0], 1, S, tabs)           # recompute
    om.layer_backward(one, P, c, g, lw, lora[0], 1, S, tabs)
    t_layer = time.perf_counter() - t0
    model = om.Model(cfg, [], None, synth.lm_head(cfg, threads=threads).float().numpy(),
                     np.ones(cfg.d, np.float32))
    ids = synth.token_ids(cfg, 1, S, seed=41)
    t1 = time.perf_counter()
    hc = om.head_forward(cfg, P, model, x)
    tgt = om.targets(ids)
    w = np.where(tgt >= 0, 1.0 / (S - 1), 0.0)
    om.head_backward(cfg, P, model, x, hc, tgt, w)
    t_head = time.perf_counter() - t1
    step = cfg.L * t_layer + t_head
    return {"value": T / step, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": (f"one 8B-shaped layer (NF4 decode, forward, recomputed forward, backward; "
                       f"{t_layer:.2f} s) and the LM head forward+backward ({t_head:.2f} s) at {T} tokens, "
                       f"mirror precision; step time scaled as {cfg.L} x layer + head = {step:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--seq", type=int, default=512)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--mode", choices=["streamed", "resident"], default="streamed")
    ap.add_argument("--absmax", choices=["dq8", "f32"], default="dq8",
                    help="store format: double-quantised absmax (112.5 MB per 8B layer, the pages' store) "
                         "or float32 absmax (122.7 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-fence", action="store_true",
                    help="copy stream waits on slot releases on the device (default: the host waits)")
    ap.add_argument("--optimizer", choices=["adamw", "adamw-separate", "none"], default="adamw",
                    help="update the LoRA vector with AdamW (lr 2e-5, the pages' config) inside every timed step: "
                         "folded into the backward sweep (adamw) or as a separate call after it")
    ap.add_argument("--dpo", action="store_true", help="same as --pref dpo")
    ap.add_argument("--pref", nargs="*", default=[], choices=["dpo", "simpo", "orpo", "kto"],
                    help="also time preference steps of these heads (2 x seq, shared 128-token prompt)")
    ap.add_argument("--threads", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--disk-layers", type=int, default=0,
                    help="spill the last N layers of the store to a file (the disk tier)")
    ap.add_argument("--disk-dir", default=None, help="directory of the disk-tier file (default $TMPDIR or /tmp)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a device buffer of this many MiB 3 times and exit: the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer store streams into a single MI355X; "
              "runs on more than one GPU are not implemented", file=sys.stderr)
        sys.exit(2)
    import threading

    import numpy as np
    import torch

    import layer_streamed_qlora_block_amd as q
    import synth

    cfg = synth.LLAMA8B
    B, S = args.batch, args.seq
    T = B * S
    t_setup = time.perf_counter()
    store = build_store(q, synth, cfg, args.threads, args.absmax, args.disk_layers, args.disk_dir)
    print(f"[bench] store built: {cfg.L} x {store.record_bytes} B in {time.perf_counter() - t_setup:.1f} s",
          file=sys.stderr, flush=True)
    emb = synth.embedding(cfg, threads=args.threads).cuda()
    lm = synth.lm_head(cfg, threads=args.threads).cuda()
    fn = synth.final_norm(cfg).cuda()
    lora = torch.from_numpy(synth.pack_lora(cfg, synth.lora_init(cfg))).cuda()
    grads = torch.empty_like(lora)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    ids = torch.from_numpy(synth.token_ids(cfg, B, S, seed=41 if S == 512 else 42)).cuda()
    mode = q.QLS_STREAMED if args.mode == "streamed" else q.QLS_RESIDENT
    max_tokens = max(T, 2 * S) if (args.dpo or args.pref) else T
    sess = q.Session(store, emb, lm, fn, max_tokens=max_tokens, max_seq=S, mode=mode, timing=True)
    if args.stream_fence:
        sess.debug(q.DBG_STREAM_FENCE)
    print(f"[bench] session ready ({sess.ws_bytes / 1e9:.2f} GB workspace), setup "
          f"{time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    opt = q.AdamW(lora, lr=2e-5) if args.optimizer != "none" else None

    def train_step():
        if args.optimizer == "adamw":
            sess.sft_step_adamw(ids, opt, grads, loss)
            return
        sess.sft_step(ids, lora, grads, loss)
        if opt is not None:
            opt.step(grads)

    for _ in range(args.warmup):
        train_step()
    torch.cuda.synchronize()
    sess.reset_stats()
    torch.cuda.synchronize()
    clock = [None]
    sampler = threading.Thread(target=lambda: (time.sleep(0.2), clock.__setitem__(0, gpu_clock_mhz())))
    t0 = time.perf_counter()
    sampler.start()   # samples the clock while the timed steps run
    for i in range(args.steps):
        train_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sampler.join()
    st = sess.stats()
    loss_v = float(loss.item())
    print(f"[bench] {args.steps} steps in {elapsed:.3f} s, loss {loss_v:.4f}", file=sys.stderr, flush=True)
    assert np.isfinite(loss_v) and bool(torch.isfinite(grads).all())

    iso = h2d_isolated_gbps(torch, store.record_bytes)
    steps = max(1, st["steps"])
    h2d_ovl = st["h2d_bytes"] / (st["copy_ms"] * 1e-3) / 1e9 if st["copy_ms"] > 0 else None
    h2d_eff = st["h2d_bytes"] / elapsed / 1e9
    kern = {}
    for key, tag, desc in (("fwd", "dq_fwd", "dequant-GEMM forward (Y = X W_nf4^T + s U B^T [+ residual])"),
                           ("dx", "dq_dx", "dequant-GEMM transposed (dX = dY W_nf4 + du A)")):
        big = (st[tag + "_big_ms"], st[tag + "_big_gflop"], st[tag + "_big_launches"])
        small = (st[tag + "_ms"] - big[0], st[tag + "_gflop"] - big[1], st[tag + "_launches"] - big[2])
        for tile, (ms, gf, n) in ((256, big), (128, small)):
            if n <= 0:
                continue
            kern[f"dq_{key}_{tile}"] = {"name": f"{desc}, {tile} x {tile} tiles", "launches": n,
                                        "ms_per_step": round(ms / steps, 3), "avg_us": round(1e3 * ms / n, 2),
                                        "tflops": round(gf / ms, 2) if ms > 0 else None}
        kern[f"dq_{key}_splitk_reduce"] = {"ms_per_step": round(st[tag + "_reduce_ms"] / steps, 3)}
    timed = {k: v for k, v in kern.items() if "launches" in v}
    dom_key = max(timed, key=lambda k: timed[k]["ms_per_step"])
    dom = timed[dom_key]
    absmax_desc = ("double-quantised absmax: 8-bit codes + float32 scale per 256 blocks" if args.absmax == "dq8"
                   else "float32 absmax")
    out = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"8B-shaped streamed QLoRA SFT step: 32 layers (hidden 4096, 32/8 heads x 128, "
                                f"SwiGLU 14336), NF4 block-64 store ({absmax_desc}, {store.record_bytes / 1e6:.1f} MB "
                                f"per layer) in pinned host memory streamed through 2 device slots, bf16 embedding + "
                                f"LM head 128256 x 4096 resident, LoRA r64 alpha16 on 7 linears"),
                   "global_batch": B, "seq_len": S, "parallelism": "single GPU", "mode": args.mode,
                   "slot_fence": "device" if args.stream_fence else "host",
                   "absmax": args.absmax, "disk_layers": args.disk_layers, "optimizer": (None if opt is None else "AdamW lr 2e-5 on the LoRA vector"
                                 + (", folded into the backward sweep" if args.optimizer == "adamw" else ""))},
        "roofline": {"bound": "mfma", "kernel": dom["name"],
                     "achieved": dom["tflops"],
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom["tflops"] / BF16_PEAK_TFLOPS, 4) if dom["tflops"] else None,
                     "traffic": (TRAFFIC_BYTES_PER_LAUNCH.get((dom_key, S)) if B == 1 else None),
                     "traffic_unit": "HBM bytes per launch"},
        "kernels": kern,
        "h2d": {"bytes_per_step": st["h2d_bytes"] // steps, "layer_loads_per_step": st["layer_loads"] / steps,
                "isolated_GBps": round(iso, 2),
                "under_overlap_GBps": round(h2d_ovl, 2) if h2d_ovl else None,
                "frac_of_isolated": round(h2d_ovl / iso, 4) if h2d_ovl else None,
                "effective_GBps": round(h2d_eff, 2),
                "effective_frac_of_isolated": round(h2d_eff / iso, 4),
                "link_theoretical_GBps": PCIE_GEN5_X16_GBPS,
                "copy_ms_per_step": round(st["copy_ms"] / steps, 3),
                "copy_overlapped_by_layer_compute": round(st["overlap_ms"] / st["copy_ms"], 4) if st["copy_ms"] else None,
                "layer_compute_ms_per_step": round(st["compute_ms"] / steps, 3)},
        "disk": ({"layers_on_disk": args.disk_layers, "reads_per_step": st["disk_reads"] / steps,
                  "read_GBps": round(st["disk_bytes"] / (st["disk_read_ms"] * 1e-3) / 1e9, 2)
                  if st["disk_read_ms"] else None,
                  "host_wait_ms_per_step": round(st["disk_wait_ms"] / steps, 3)} if args.disk_layers else None),
        "peak_hbm_GB": round(torch.cuda.max_memory_allocated() / 1e9, 3),
        "gpu_clock": clock[0],
        "loss": round(loss_v, 5),
    }
    kinds = list(dict.fromkeys((["dpo"] if args.dpo else []) + args.pref))
    if kinds:
        P = 128
        c, r = synth.dpo_pair(cfg, S, P)
        c, r = torch.from_numpy(c).cuda(), torch.from_numpy(r).cuda()
        params = {"dpo": {"beta": 0.1}, "simpo": {"beta": 2.0, "gamma": 1.0}, "orpo": {"lam": 0.1},
                  "kto": {"beta": 0.1, "lam_d": 1.0, "lam_u": 1.0}}
        out["pref"] = {}
        for kind in kinds:
            sess.pref_step(kind, c, r, P, lora, grads, loss, **params[kind])
            torch.cuda.synchronize()
            sess.reset_stats()
            t0 = time.perf_counter()
            n = max(1, args.steps // 2)
            for _ in range(n):
                sess.pref_step(kind, c, r, P, lora, grads, loss, **params[kind])
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / n
            out["pref"][kind] = {"params": params[kind], "ms_per_step": round(1e3 * dt, 3),
                                 "tokens_per_s": round(2 * S / dt, 2),
                                 "layer_loads_per_step": sess.stats()["layer_loads"] / n,
                                 "loss": float(loss.item())}
    sess.close()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(synth, cfg, T, args.threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
