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
peak device memory, and the CPU oracle timed on a bounded sample.  Unless
``--no-extra``, the line also carries two further workloads timed after the
headline: the DPO step on the same stack (chosen and rejected 1 x 512 sharing
a 128-token prompt) and the SFT step at seq 4096.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "streamed QLoRA SFT tokens/sec (8B-shape, seq 512); % H2D BW and % MFMA peak"
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PCIE_GEN5_X16_GBPS = 64.0       # theoretical per direction
# HBM bytes per launch of the forward dequant-GEMM come from rocprofv3
# FETCH_SIZE / WRITE_SIZE passes scaled by a known-size copy, summarised in this
# profile with the hash of the kernel and launch-plan sources they were taken
# on; a figure whose hash no longer matches the sources is reported as null.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_dequant_gemm_8b.md")
KERNEL_SOURCES = ("layer_streamed_qlora_block_amd/csrc/gemm_big.hip", "layer_streamed_qlora_block_amd/csrc/ops.cpp")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(seq):
    """(bytes per launch, note) of the forward dequant-GEMM at this sequence
    length from the committed counter summary, or (None, why)."""
    try:
        lines = open(TRAFFIC_PROFILE).read().splitlines()
    except OSError:
        return None, "no counter summary"
    cur = kernel_source_hash()
    for ln in lines:
        if not ln.startswith("traffic-record: "):
            continue
        rec = json.loads(ln[len("traffic-record: "):])
        if rec.get("seq") != seq:
            continue
        if rec.get("source_sha256_16") != cur:
            return None, f"counters taken on other kernel sources ({rec.get('source_sha256_16')} != {cur})"
        return rec["bytes_per_launch"], f"rocprofv3 FETCH_SIZE + WRITE_SIZE, {os.path.basename(TRAFFIC_PROFILE)}"
    return None, f"no counter record for seq {seq}"


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


def h2d_isolated_gbps(torch, store, iters=20):
    """Median rate of hipMemcpyAsync copies of layer 0's pinned record (the
    store's own hipHostMalloc memory, as the stream copies it) into a device
    buffer, one at a time on an otherwise idle stream."""
    import ctypes
    view = store.view(0)
    nbytes = int(view.record_bytes)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    times = []
    for i in range(iters + 2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        rc = hip.hipMemcpyAsync(dst.data_ptr(), view.record, nbytes, 1, s.cuda_stream)   # 1: host to device
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed: {rc}")
        b.record(s)
        b.synchronize()
        if i >= 2:
            times.append(a.elapsed_time(b))
    times.sort()
    return nbytes / (times[len(times) // 2] * 1e-3) / 1e9


def summarize_trace(d, record_bytes, steps):
    """Markdown summary of a rocprofv3 --kernel-trace --memory-copy-trace run
    (CSV files under d): time per kernel, the host-to-device copies (whole
    layer records told apart from the part copies by duration), and the copy /
    kernel overlap from the trace timestamps."""
    import csv
    import glob

    def rows(pat):
        out = []
        for f in sorted(glob.glob(os.path.join(d, "**", pat), recursive=True)):
            with open(f, newline="") as fh:
                out += list(csv.DictReader(fh))
        return out

    def short(name):
        n = name.replace("(anonymous namespace)::", "")
        if n.startswith("void "):
            n = n[5:]
        depth = 0
        for i, ch in enumerate(n):          # cut the argument list at template depth 0
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
            elif ch == "(" and depth == 0:
                return n[:i]
        return n

    ours = ("embed_k", "big_kernel", "gemm_kernel", "reduce", "attn_", "rmsnorm", "rope_", "swiglu", "adamw",
            "lora_cast", "ce_", "sft_loss", "absmax_expand", "pref_k", "seq_logp", "group_sum")
    kr = [dict(r, name=short(r["Kernel_Name"])) for r in rows("*kernel_trace.csv")]
    step_k = [r for r in kr if r["name"].startswith(ours)]
    if not step_k:
        raise SystemExit(f"no kernel of the step in the trace under {d}")
    # The window of the steps: from the first embedding gather to the last
    # kernel of the library (setup uploads and the later isolated copies fall
    # outside it).
    w0 = min(int(r["Start_Timestamp"]) for r in step_k if r["name"].startswith("embed_k"))
    w1 = max(int(r["End_Timestamp"]) for r in step_k)
    kr = [r for r in kr if int(r["Start_Timestamp"]) >= w0 and int(r["End_Timestamp"]) <= w1]
    cr = [r for r in rows("*memory_copy_trace.csv") if r.get("Direction", "").endswith("HOST_TO_DEVICE")
          and int(r["Start_Timestamp"]) >= w0 and int(r["End_Timestamp"]) <= w1]
    kint = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in kr)
    per = {}
    for r in kr:
        n = r["name"]
        a = per.setdefault(n, [0, 0])
        a[0] += 1
        a[1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    busy = []                                   # union of kernel intervals
    for a, b in kint:
        if busy and a <= busy[-1][1]:
            busy[-1][1] = max(busy[-1][1], b)
        else:
            busy.append([a, b])
    total_k = sum(v[1] for v in per.values())
    lines = [f"Window of the {steps} steps: {(w1 - w0) / 1e6:.2f} ms ({(w1 - w0) / 1e6 / steps:.2f} ms per step).",
             f"Kernels: {len(kr)} dispatches, {total_k / 1e6:.2f} ms of kernel time over {steps} steps "
             f"({total_k / 1e6 / steps:.2f} ms per step); the GPU runs at least one kernel for "
             f"{sum(b - a for a, b in busy) / 1e6 / steps:.2f} ms per step.", "",
             "| kernel | calls | total ms | ms / step | avg us | % |", "|---|---:|---:|---:|---:|---:|"]
    for n, (c, t) in sorted(per.items(), key=lambda kv: -kv[1][1])[:25]:
        lines.append(f"| `{n}` | {c} | {t / 1e6:.2f} | {t / 1e6 / steps:.2f} | {t / 1e3 / c:.1f} | "
                     f"{100 * t / total_k:.2f} |")
    if cr:
        import bisect
        cint = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in cr)
        starts = [a for a, _ in busy]

        def covered(a, b):
            i = max(0, bisect.bisect_right(starts, a) - 1)
            tot = 0
            while i < len(busy) and busy[i][0] < b:
                tot += max(0, min(b, busy[i][1]) - max(a, busy[i][0]))
                i += 1
            return tot

        dur = [b - a for a, b in cint]
        ov = [covered(a, b) for a, b in cint]
        whole = sorted(x for x in dur if x > 1.5e6)
        tot_c, tot_o = sum(dur), sum(ov)
        lines += ["", f"Host-to-device copies: {len(cint)} ({len(whole)} whole layer records of {record_bytes} B, "
                  f"longer than 1.5 ms; the rest are the part copies of the first copy of each sweep), "
                  f"{tot_c / 1e6 / steps:.2f} ms of copy time per step."]
        if whole:
            gb = sorted(record_bytes / (x * 1e-9) / 1e9 for x in whole)
            q = lambda p: gb[min(len(gb) - 1, int(p * len(gb)))]
            lines.append(f"Whole-record copies: median {q(0.5):.2f} GB/s (p10 {q(0.1):.2f}, p90 {q(0.9):.2f}), "
                         f"median duration {whole[len(whole) // 2] / 1e6:.3f} ms.")
        lines.append(f"Copy / kernel overlap from the trace timestamps: {100 * tot_o / max(tot_c, 1):.1f}% of "
                     f"the copy time has a kernel running; exposed copy time (no kernel running) "
                     f"{(tot_c - tot_o) / 1e6 / steps:.2f} ms per step.")
    return "\n".join(lines)


def summarize_counters(d, kernel_regex):
    """Average of every counter of a rocprofv3 --pmc run (CSV files under d)
    per dispatch of the kernels whose name matches kernel_regex."""
    import csv
    import glob
    import re
    rx = re.compile(kernel_regex)
    per = {}
    dur = {}                                       # dispatch -> ns, from the rows' timestamps
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                if not rx.search(name):
                    continue
                per.setdefault(r.get("Counter_Name"), {}).setdefault(r.get("Dispatch_Id"), 0.0)
                per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r.get("Counter_Value", 0) or 0)
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    lines = [f"Kernels matching `{kernel_regex}` under {os.path.basename(os.path.normpath(d))}:", "",
             "| counter | dispatches | average per dispatch |", "|---|---:|---:|"]
    for c, vals in sorted(per.items()):
        v = list(vals.values())
        lines.append(f"| {c} | {len(v)} | {sum(v) / len(v):.1f} |")
    if dur:
        lines.append(f"| duration (us, from the dispatch timestamps) | {len(dur)} | "
                     f"{sum(dur.values()) / len(dur) / 1e3:.1f} |")
    return "\n".join(lines)


class _LazyLayers:
    """Oracle model layers that decode their NF4 codes on every access, as the
    method decodes each streamed layer it uses (store build untimed)."""

    def __init__(self, cfg, store):
        self.cfg, self.store = cfg, store
        self.ones = None

    def __len__(self):
        return len(self.store)

    def __getitem__(self, l):
        import numpy as np
        from oracle import model as om
        from oracle import nf4
        shapes = [(o, i) for _, o, i in self.cfg.module_shapes()]
        W = {n: nf4.dequant(c, a, sh) for n, (c, a), sh in zip(om.NAMES, self.store[l], shapes)}
        ones = np.ones(self.cfg.d, np.float32)
        return {"W": W, "norm_attn": ones, "norm_mlp": ones}


def cpu_info():
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        b = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if b:
            blas = f"{b[0].get('internal_api')} {b[0].get('version')} ({b[0].get('architecture')})"
    except Exception:
        pass
    return model, blas


def cpu_baseline(synth, cfg, S, threads, dpo=True):
    """The oracle, untouched (mirror precision), on full steps of 1- and
    2-layer 8B-shaped stacks: embedding, forward sweep, LM head (forward and
    backward), backward sweep with recompute, NF4 decode on every layer use.
    The 32-layer time is t1 + 31 (t2 - t1).  The same for the DPO step."""
    import numpy as np
    from oracle import model as om
    from oracle import nf4
    from threadpoolctl import threadpool_limits
    threadpool_limits(threads)
    two = synth.scaled(cfg, L=2)
    with cf.ThreadPoolExecutor(7) as ex:                 # store build: untimed
        store = [list(ex.map(nf4.quantize, synth.base_layer(two, l, threads=threads))) for l in range(2)]
    emb = synth.embedding(cfg, threads=threads).float().numpy()
    lm = synth.lm_head(cfg, threads=threads).float().numpy()
    P = om.Prec("mirror")
    ids = synth.token_ids(cfg, 1, S, seed=41 if S == 512 else 42)
    c, r = synth.dpo_pair(cfg, S, 128)
    times = {"sft": {}, "dpo": {}}
    for L in (1, 2):
        cl = synth.scaled(cfg, L=L)
        model = om.Model(cl, _LazyLayers(cl, store[:L]), emb, lm, np.ones(cfg.d, np.float32))
        lora = synth.lora_init(cl)
        t0 = time.perf_counter()
        om.sft_step(cl, P, model, lora, ids)
        times["sft"][L] = time.perf_counter() - t0
        if dpo:
            t0 = time.perf_counter()
            om.dpo_step(cl, P, model, lora, c, r, 128, 0.1)
            times["dpo"][L] = time.perf_counter() - t0
    model_name, blas = cpu_info()
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count()

    def scale(t):
        return t[1] + (cfg.L - 1) * (t[2] - t[1])

    sft = scale(times["sft"])
    out = {"value": S / sft, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"full oracle SFT steps (mirror precision: embedding, forward sweep, LM head forward and "
                      f"backward, backward sweep with recompute, NF4 decode on every layer use) on 1- and 2-layer "
                      f"8B-shaped stacks at batch 1 x {S}: {times['sft'][1]:.1f} s and {times['sft'][2]:.1f} s; "
                      f"32-layer step time extrapolated as t1 + 31 (t2 - t1) = {sft:.1f} s"),
           "cpu_model": model_name, "blas": blas, "affinity_cpus": aff,
           "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    if dpo:
        d = scale(times["dpo"])
        out["dpo"] = {"value": 2 * S / d, "unit": "tokens/s", "step_s": round(d, 2),
                      "sample": (f"oracle DPO steps (reference pass, policy pass, backward) on the 1- and 2-layer "
                                 f"stacks: {times['dpo'][1]:.1f} s and {times['dpo'][2]:.1f} s, extrapolated to 32 "
                                 f"layers")}
    return out


def kernel_summary(st, steps):
    kern = {}
    for key, tag, desc in (("fwd", "dq_fwd", "dequant-GEMM forward (Y = X W_nf4^T + s U B^T [+ residual])"),
                           ("dx", "dq_dx", "dequant-GEMM transposed (dX = dY W_nf4 + du A)")):
        big = (st[tag + "_big_ms"], st[tag + "_big_gflop"], st[tag + "_big_launches"], st[tag + "_big_reduce_ms"])
        small = (st[tag + "_ms"] - big[0], st[tag + "_gflop"] - big[1], st[tag + "_launches"] - big[2],
                 st[tag + "_reduce_ms"] - big[3])
        for tile, (ms, gf, n, red) in ((256, big), (128, small)):
            if n <= 0:
                continue
            kern[f"dq_{key}_{tile}"] = {"name": f"{desc}, {tile} x {tile} tiles", "launches": n,
                                        "ms_per_step": round(ms / steps, 3), "avg_us": round(1e3 * ms / n, 2),
                                        "tflops": round(gf / ms, 2) if ms > 0 else None,
                                        "splitk_reduce_ms_per_step": round(red / steps, 3),
                                        "tflops_incl_splitk_reduce": round(gf / (ms + red), 2) if ms > 0 else None}
    return kern


def roofline(kern, key, seq, batch):
    dom = kern[key]
    traffic, note = measured_traffic(seq) if (batch == 1 and key == "dq_fwd_256") else (None, "not measured")
    return {"bound": "mfma", "kernel": dom["name"], "achieved": dom["tflops"], "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(dom["tflops"] / BF16_PEAK_TFLOPS, 4) if dom["tflops"] else None,
            "traffic": traffic, "traffic_unit": "HBM bytes per launch", "traffic_source": note,
            "achieved_incl_splitk_reduce": dom["tflops_incl_splitk_reduce"],
            "frac_incl_splitk_reduce": (round(dom["tflops_incl_splitk_reduce"] / BF16_PEAK_TFLOPS, 4)
                                        if dom["tflops_incl_splitk_reduce"] else None)}


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
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the DPO and seq-4096 workloads timed after the headline")
    ap.add_argument("--stream-fence", action="store_true",
                    help="copy stream waits on slot releases on the device (default: the host waits)")
    ap.add_argument("--optimizer", choices=["adamw", "adamw-separate", "none"], default="adamw",
                    help="update the LoRA vector with AdamW (lr 2e-5, the pages' config) inside every timed step: "
                         "folded into the backward sweep (adamw) or as a separate call after it")
    ap.add_argument("--pref", nargs="*", default=[], choices=["dpo", "simpo", "orpo", "kto"],
                    help="also time preference steps of these heads (2 x seq, shared 128-token prompt)")
    ap.add_argument("--threads", type=int, default=None,
                    help="host threads for the store build and the CPU oracle (default: the CPUs of this "
                         "process's affinity mask, at most OMP_NUM_THREADS when that is set)")
    ap.add_argument("--disk-layers", type=int, default=0,
                    help="spill the last N layers of the store to a file (the disk tier)")
    ap.add_argument("--disk-dir", default=None, help="directory of the disk-tier file (default $TMPDIR or /tmp)")
    ap.add_argument("--summarize-trace", default=None, metavar="DIR",
                    help="only print a markdown summary of the rocprofv3 kernel / memory-copy trace CSVs under DIR")
    ap.add_argument("--trace-steps", type=int, default=1, help="steps the summarised trace covers")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR",
                    help="only print the per-dispatch average of every rocprofv3 --pmc counter under DIR for the "
                         "kernels matching --kernel-regex")
    ap.add_argument("--kernel-regex", default=r"big_kernel<2, 0>", help="kernel name pattern for --summarize-counters")
    ap.add_argument("--record-bytes", type=int, default=112529408,
                    help="bytes of one layer record in the summarised trace (default: the dq8 8B record)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only copy a device buffer of this many MiB 3 times and exit: the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.record_bytes, args.trace_steps))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.kernel_regex))
        return
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
    if args.threads is None:
        try:
            aff = len(os.sched_getaffinity(0))
        except AttributeError:
            aff = os.cpu_count() or 1
        omp = os.environ.get("OMP_NUM_THREADS", "")
        args.threads = min(aff, int(omp)) if omp.isdigit() and int(omp) > 0 else aff
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
    extra = not args.no_extra and S == 512 and B == 1
    max_tokens = max(T, 2 * S) if (args.pref or extra) else T
    sess = q.Session(store, emb, lm, fn, max_tokens=max_tokens, max_seq=S, mode=mode, timing=True)
    if args.stream_fence:
        sess.debug(q.DBG_STREAM_FENCE)
    print(f"[bench] session ready ({sess.ws_bytes / 1e9:.2f} GB workspace), setup "
          f"{time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    opt = q.AdamW(lora, lr=2e-5) if args.optimizer != "none" else None

    def train_step(sess_, ids_):
        if args.optimizer == "adamw":
            sess_.sft_step_adamw(ids_, opt, grads, loss)
            return
        sess_.sft_step(ids_, lora, grads, loss)
        if opt is not None:
            opt.step(grads)

    def timed_sft(sess_, ids_, steps, warmup):
        for _ in range(warmup):
            train_step(sess_, ids_)
        torch.cuda.synchronize()
        sess_.reset_stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            train_step(sess_, ids_)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    clock = [None]
    sampler = threading.Thread(target=lambda: (time.sleep(0.2), clock.__setitem__(0, gpu_clock_mhz())))
    sampler.start()   # samples the clock while the timed steps run
    elapsed = timed_sft(sess, ids, args.steps, args.warmup)
    sampler.join()
    st = sess.stats()
    loss_v = float(loss.item())
    print(f"[bench] {args.steps} steps in {elapsed:.3f} s, loss {loss_v:.4f}", file=sys.stderr, flush=True)
    assert np.isfinite(loss_v) and bool(torch.isfinite(grads).all())

    iso = h2d_isolated_gbps(torch, store)
    steps = max(1, st["steps"])
    h2d_ovl = st["h2d_bytes"] / (st["copy_ms"] * 1e-3) / 1e9 if st["copy_ms"] > 0 else None
    h2d_eff = st["h2d_bytes"] / elapsed / 1e9
    kern = kernel_summary(st, steps)
    timed = {k: v for k, v in kern.items() if "launches" in v}
    dom_key = max(timed, key=lambda k: timed[k]["ms_per_step"])
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
                   "absmax": args.absmax, "disk_layers": args.disk_layers,
                   "optimizer": (None if opt is None else "AdamW lr 2e-5 on the LoRA vector"
                                 + (", folded into the backward sweep" if args.optimizer == "adamw" else ""))},
        "roofline": roofline(kern, dom_key, S, B),
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
                "exposed_copy_ms_per_step": round(st["exposed_copy_ms"] / steps, 3),
                "layer_compute_ms_per_step": round(st["compute_ms"] / steps, 3)},
        "disk": ({"layers_on_disk": args.disk_layers, "reads_per_step": st["disk_reads"] / steps,
                  "read_GBps": round(st["disk_bytes"] / (st["disk_read_ms"] * 1e-3) / 1e9, 2)
                  if st["disk_read_ms"] else None,
                  "host_wait_ms_per_step": round(st["disk_wait_ms"] / steps, 3)} if args.disk_layers else None),
        "peak_hbm_GB": round(torch.cuda.max_memory_allocated() / 1e9, 3),
        "peak_ws_GB": round(st["peak_ws_bytes"] / 1e9, 3),
        "gpu_clock": clock[0],
        "loss": round(loss_v, 5),
    }
    P = 128
    kinds = list(dict.fromkeys((["dpo"] if extra else []) + args.pref))
    if kinds:
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
            n = max(2, args.steps // 2)
            for _ in range(n):
                sess.pref_step(kind, c, r, P, lora, grads, loss, **params[kind])
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / n
            pst = sess.stats()
            out["pref"][kind] = {"workload": (f"{kind.upper()} step on the same streamed stack: chosen and rejected "
                                              f"1 x {S} sharing a {P}-token prompt"),
                                 "params": params[kind], "ms_per_step": round(1e3 * dt, 3),
                                 "tokens_per_s": round(2 * S / dt, 2),
                                 "layer_loads_per_step": pst["layer_loads"] / n,
                                 "h2d_GBps_under_overlap": (round(pst["h2d_bytes"] / (pst["copy_ms"] * 1e-3) / 1e9, 2)
                                                            if pst["copy_ms"] else None),
                                 "loss": float(loss.item())}
    sess.close()
    if extra:
        # The long-sequence SFT step: compute-bound, the dequant-GEMM at 4096 tokens.
        S4 = 4096
        sess4 = q.Session(store, emb, lm, fn, max_tokens=S4, max_seq=S4, mode=mode, timing=True)
        ids4 = torch.from_numpy(synth.token_ids(cfg, 1, S4, seed=42)).cuda()
        n4 = max(3, args.steps // 4)
        el4 = timed_sft(sess4, ids4, n4, 1)
        st4 = sess4.stats()
        k4 = kernel_summary(st4, max(1, st4["steps"]))
        t4 = {k: v for k, v in k4.items() if "launches" in v}
        dom4 = max(t4, key=lambda k: t4[k]["ms_per_step"])
        out["sft_seq4096"] = {
            "workload": "the same streamed 8B-shaped SFT step at batch 1 x seq 4096 (token ids seed 42)",
            "tokens_per_s": round(S4 * n4 / el4, 2), "ms_per_step": round(1e3 * el4 / n4, 3), "steps": n4,
            "warmup": 1, "roofline": roofline(k4, dom4, S4, 1), "kernels": k4,
            "copy_overlapped_by_layer_compute": round(st4["overlap_ms"] / st4["copy_ms"], 4) if st4["copy_ms"] else None,
            "exposed_copy_ms_per_step": round(st4["exposed_copy_ms"] / max(1, st4["steps"]), 3),
            "peak_hbm_GB": round(torch.cuda.max_memory_allocated() / 1e9, 3), "loss": round(float(loss.item()), 5)}
        sess4.close()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(synth, cfg, S, args.threads, dpo=extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
