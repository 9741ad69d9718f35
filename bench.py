#!/usr/bin/env python3
"""Benchmark of the vocab-wide softmax hot path on one MI355X.

One step = forward + backward of the four per-token ops the pages measure
(DeepSpeed PR #8838, first and second commit messages) on the 8192 x 75968
bf16 logit pair:
    logprobs(A), entropy(A), KL(A||B) (grads to A and B), KL(B||A) (grads to B and A).
Inputs are generated on the host (seeded, vocab_wide_softmax_amd.workloads),
copied to HBM before timing, and every step reruns all eight kernel launches
(plus nothing else) through the C ABI.

Printed: one JSON line with the step throughput in algorithmic GB/s (bytes the
single-read method must move: 18 x 1.2447 GB per step), ms per step, the
per-op split (from an untimed pass with events around every launch), a roofline
object for the dominant kernel (the KL(A||B) backward, bracketed by HIP events
on its stream inside the timed steps), and the fp64 oracle's throughput on a
bounded sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --calibrate          # plain copies of known size, for counter scaling
    python bench.py --summarize DIR stats|counters   # condense rocprofv3 output for profiles/
    python bench.py --counters FETCH WRITE CALFETCH CALWRITE   # calibrated HBM bytes per kernel
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd ms + achieved HBM GB/s (% of peak), 8192×75968 bf16 KL/entropy/logp"
PEAK_GBS = 8000.0
N_ROWS, V = 8192, 75968
T_BYTES = N_ROWS * V * 2  # one bf16 [8192, 75968] tensor
# algorithmic bytes per op (fwd + bwd): logprobs/entropy 1 read + (1 read + 1 write);
# KL with both gradients 2 reads + (2 reads + 2 writes)
OP_BYTES = {"logprobs": 3 * T_BYTES, "entropy": 3 * T_BYTES, "kl_ab": 6 * T_BYTES, "kl_ba": 6 * T_BYTES}
STEP_BYTES = sum(OP_BYTES.values())
DOMINANT = "kl_bwd"  # KL backward: reads A and B, writes dA and dB
DOMINANT_BYTES = 4 * T_BYTES
DOM_PHASE = "kl_ab_bwd"  # the launch of it that the timed steps bracket with events
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["vocab_wide_softmax_amd/csrc/bwd.hip", "vocab_wide_softmax_amd/csrc/device.h"]


def kernel_source_hash():
    """Hash of the dominant kernel's code with // comments and blank lines removed, so that
    the stored counter figures stay valid across comment-only edits and no longer."""
    import re

    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            src = re.sub(r"//[^\n]*", "", f.read())
        h.update("\n".join(line.rstrip() for line in src.split("\n") if line.strip()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    or None when it is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, "kl_bwd_pair8192_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- GPU step

def make_inputs(wl, device):
    import torch

    from vocab_wide_softmax_amd import workloads as W

    a, b, t = wl.a.to(device), wl.b.to(device), wl.t.to(device)
    g = {op: wl.g[op].to(device) for op in W.OPS}
    torch.cuda.synchronize()
    return wl, a, b, t, g


def run_step(B, a, b, t, g, ev=None, split=0):
    """One pass of the hot path. ev: optional dict of (start, end) event lists per op phase."""
    import torch

    stream = torch.cuda.current_stream()

    def rec(key, i):
        if ev is not None and key in ev:
            ev[key][i].record(stream)

    rec("logprobs_fwd", 0)
    lp, st = B.logprobs_fwd(a, t, -100, split)
    rec("logprobs_fwd", 1)
    rec("logprobs_bwd", 0)
    B.logprobs_bwd(a, t, st, g["logprobs"], -100)
    rec("logprobs_bwd", 1)
    rec("entropy_fwd", 0)
    H, st = B.entropy_fwd(a, split)
    rec("entropy_fwd", 1)
    rec("entropy_bwd", 0)
    B.entropy_bwd(a, st, H, g["entropy"])
    rec("entropy_bwd", 1)
    for name, x, y in (("kl_ab", a, b), ("kl_ba", b, a)):
        rec(name + "_fwd", 0)
        kl, st = B.kl_fwd(x, y, split)
        rec(name + "_fwd", 1)
        rec(name + "_bwd", 0)
        B.kl_bwd(x, y, st, kl, g[name])
        rec(name + "_bwd", 1)


PHASES = ["logprobs_fwd", "logprobs_bwd", "entropy_fwd", "entropy_bwd", "kl_ab_fwd", "kl_ab_bwd", "kl_ba_fwd",
          "kl_ba_bwd"]


def gpu_bench(wl, steps, warmup, device):
    """Warm up, then time exactly `steps` steps (synchronised on both sides). Inside the timed
    steps HIP events bracket only the dominant kernel (the KL(A||B) backward), on the stream it is
    launched on; a second, untimed pass of `steps` steps with events around every phase gives the
    per-op breakdown (each event pair costs a few microseconds, so the timed steps carry only one)."""
    import torch

    from vocab_wide_softmax_amd import binding as B

    B.lib()
    wl, a, b, t, g = make_inputs(wl, device)
    log("inputs resident in HBM; %d warmup steps" % warmup)
    for _ in range(warmup):
        run_step(B, a, b, t, g)

    def events(keys):
        return [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in keys}
                for _ in range(steps)]

    dom = events([DOM_PHASE])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(B, a, b, t, g, dom[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    dom_ms = [ev[DOM_PHASE][0].elapsed_time(ev[DOM_PHASE][1]) for ev in dom]

    evs = events(PHASES)
    for i in range(steps):
        run_step(B, a, b, t, g, evs[i])
    torch.cuda.synchronize()
    per = {k: [ev[k][0].elapsed_time(ev[k][1]) for ev in evs] for k in PHASES}
    med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
    return ms_per_step, med, sum(dom_ms) / len(dom_ms)


# ------------------------------------------------------------------------- other ops

def _timed(fwd, bwd, steps, warmup):
    """Median fwd and bwd milliseconds (HIP events on the current stream). All steps are
    enqueued before one synchronisation, so the host runs ahead and an event interval holds
    the kernels only, not the host work of issuing them."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bwd(fwd())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record(stream)
        r = fwd()
        e[1].record(stream)
        bwd(r)
        e[2].record(stream)
    torch.cuda.synchronize()
    f = sorted(e[0].elapsed_time(e[1]) for e in evs)
    b = sorted(e[1].elapsed_time(e[2]) for e in evs)
    return f[steps // 2], b[steps // 2]


def extras_bench(wl, device, steps=15, warmup=30):
    """The other ops on the same 8192 x 75968 pair, each fwd+bwd, with their algorithmic bytes:
    top-k logprobs (K = 16 ids per row), the generalized JSD (beta = 0.5: two reads of both
    inputs forward, one read of both and two writes backward), the four-op step on fp16 copies
    of the logits, and the four-op step in the batch-invariant split mode. These legs start right
    after their inputs' host-to-device copies, when the card runs its first few dozen sub-ms
    kernels slower (top-k backward 0.47 ms there, 0.39 ms afterwards); each leg therefore warms
    up with 30 untimed calls before its 15 timed ones."""
    import torch

    from vocab_wide_softmax_amd import binding as B
    from vocab_wide_softmax_amd import workloads as W

    a, b = wl.a.to(device), wl.b.to(device)
    g = {op: wl.g[op].to(device) for op in W.OPS}
    ids = torch.randint(0, V, (N_ROWS, 16), generator=torch.Generator().manual_seed(5)).to(device)
    gk = torch.randn(N_ROWS, 16, generator=torch.Generator().manual_seed(6)).to(device)
    torch.cuda.synchronize()
    out = {}

    def put(name, f_ms, b_ms, nbytes):
        gbs = nbytes / ((f_ms + b_ms) * 1e-3) / 1e9
        out[name] = {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "fwd_bwd_ms": round(f_ms + b_ms, 4),
                     "bytes": nbytes, "GB/s": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_GBS, 1)}

    f_ms, b_ms = _timed(lambda: B.logprobs_topk_fwd(a, ids, -100),
                        lambda r: B.logprobs_topk_bwd(a, ids, r[1], gk, -100), steps, warmup)
    put("logprobs_topk16", f_ms, b_ms, 3 * T_BYTES)
    f_ms, b_ms = _timed(lambda: B.jsd_fwd(a, b, 0.5),
                        lambda r: B.jsd_bwd(a, b, 0.5, r[1], r[0], g["kl_ab"]), steps, warmup)
    put("jsd_beta0.5", f_ms, b_ms, 8 * T_BYTES)
    t = wl.t.to(device)
    for name, x, y, split in (("step_fp16", a.half(), b.half(), 0), ("step_batch_invariant", a, b, -1)):
        torch.cuda.synchronize()
        for _ in range(warmup):
            run_step(B, x, y, t, g, split=split)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step(B, x, y, t, g, split=split)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        gbs = STEP_BYTES / (ms * 1e-3) / 1e9
        out[name] = {"ms_per_step": round(ms, 4), "bytes": STEP_BYTES, "GB/s": round(gbs, 1),
                     "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
    return out


# ------------------------------------------------------------------- fused linear-logp

LIN_N, LIN_H, LIN_V = 8192, 4096, 151936
MFMA_BF16_PEAK_TFLOPS = 2500.0


def linear_bench(steps, warmup, device):
    """Forward + backward of the fused linear-logp on h [8192, 4096], W [151936, 4096] bf16.
    FLOPs counted: forward 2 N H V; backward 3 x 2 N H V (logits recomputed, dh, dW)."""
    import torch

    from vocab_wide_softmax_amd import binding as B
    from vocab_wide_softmax_amd import workloads as W

    wl = W.linear_logp(LIN_N, LIN_H, LIN_V)
    h, Wm, t, g = wl.h.to(device), wl.W.to(device), wl.t.to(device), wl.g.to(device)
    torch.cuda.synchronize()
    log("linear-logp inputs resident; %d warmup steps" % warmup)
    for _ in range(warmup):
        lp, st = B.linear_logp_fwd(h, Wm, t)
        B.linear_logp_bwd(h, Wm, t, st, g)
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        lp, st = B.linear_logp_fwd(h, Wm, t)
        evs[i][1].record(stream)
        B.linear_logp_bwd(h, Wm, t, st, g)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    fwd = sorted(e[0].elapsed_time(e[1]) for e in evs)[steps // 2]
    bwd = sorted(e[1].elapsed_time(e[2]) for e in evs)[steps // 2]
    flop = 2.0 * LIN_N * LIN_H * LIN_V
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    return {
        "workload": "h [8192, 4096] ~ N(0,1), W [151936, 4096] ~ N(0, 0.02^2), bf16; targets U[0, 151936)",
        "ms_per_step": round(wall, 3), "fwd_ms": round(fwd, 3), "bwd_ms": round(bwd, 3),
        "fwd_tflops": round(tf(flop, fwd), 1), "bwd_tflops": round(tf(3 * flop, bwd), 1),
        "step_tflops": round(tf(4 * flop, fwd + bwd), 1),
        "roofline": {"bound": "mfma", "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf(4 * flop, fwd + bwd) / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


# --------------------------------------------------------------------------- CPU oracle

def _oracle_rows(args):
    import numpy as np

    from oracle import reductions as R

    a, b, t, gs = args
    R.logprobs_fwd(a, t)
    R.logprobs_bwd(a, t, gs[0])
    R.entropy_fwd(a)
    R.entropy_bwd(a, gs[1])
    R.kl_fwd(a, b)
    R.kl_bwd(a, b, gs[2])
    R.kl_fwd(b, a)
    R.kl_bwd(b, a, gs[3])
    return int(np.asarray(a).shape[0])


def cpu_baseline(wl, rows=8192):
    """The fp64 oracle on `rows` rows of the same workload, row chunks spread over host
    threads (numpy releases the GIL inside its array kernels)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from vocab_wide_softmax_amd import workloads as W

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    idx = np.linspace(0, N_ROWS - 1, rows).astype(np.int64)
    a = wl.a[idx].double().numpy()
    b = wl.b[idx].double().numpy()
    t = wl.t[idx].numpy()
    gs = [wl.g[op][idx].double().numpy() for op in W.OPS]
    chunks = [c for c in np.array_split(np.arange(rows), rows // 4 if rows >= 4 else 1) if len(c)]
    work = [(a[c], b[c], t[c], [x[c] for x in gs]) for c in chunks]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        done = sum(ex.map(_oracle_rows, work))
    el = time.perf_counter() - t0
    assert done == rows
    bytes_sample = STEP_BYTES * rows / N_ROWS
    return {
        "value": round(bytes_sample / el / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d of 8192 rows (evenly spaced) of the 8192x75968 bf16 pair, all four ops fwd+bwd in float64 "
                  "on %d host threads; %.1f s wall; GB/s = algorithmic bytes of those rows / wall time"
                  % (rows, cores, el),
    }


# ------------------------------------------------------------------------- calibration

def calibrate(device):
    """Plain device copies of a known size (1.2447 GB each way), for scaling HBM counters."""
    import torch

    src = torch.empty(T_BYTES, dtype=torch.uint8, device=device)
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_each_way": T_BYTES, "launches": 5}))


# -------------------------------------------------------------------- profile summaries

def _rocpd(outdir):
    import sqlite3

    paths = sorted(glob.glob(os.path.join(outdir, "**", "*_results.db"), recursive=True))
    if not paths:
        raise FileNotFoundError("no rocprofv3 *_results.db under " + outdir)
    return sqlite3.connect(paths[0])


def summarize(outdir, mode):
    """Condense rocprofv3 output (its SQLite database) in `outdir` into a text table.

    mode "stats": calls and average / total duration per kernel;
    mode "counters": mean value per dispatch of every collected counter, per kernel.
    """
    con = _rocpd(outdir)
    if mode == "stats":
        rows = con.execute("select name, count(*), avg(end - start), min(end - start), max(end - start), "
                           "sum(end - start) from kernels group by name order by sum(end - start) desc").fetchall()
        total = sum(r[5] for r in rows)
        print("| kernel | calls | average us | min us | max us | total us | % |")
        print("|---|---|---|---|---|---|---|")
        for name, calls, avg, mn, mx, tot in rows:
            print("| %s | %d | %.1f | %.1f | %.1f | %.1f | %.2f |" % (name, calls, avg / 1e3, mn / 1e3, mx / 1e3,
                                                                      tot / 1e3, 100.0 * tot / total))
        return
    rows = con.execute("select * from counters_collection").fetchall()
    cols = [d[0] for d in con.execute("select * from counters_collection limit 1").description]
    ci = {c: i for i, c in enumerate(cols)}
    name_col = "kernel_name" if "kernel_name" in ci else "name"
    acc = {}
    for r in rows:
        key = (r[ci[name_col]], r[ci["counter_name"]])
        acc.setdefault(key, {}).setdefault(r[ci["dispatch_id"]], 0.0)
        acc[key][r[ci["dispatch_id"]]] += float(r[ci["value"]])
    print("| kernel | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|")
    for (name, ctr), per in sorted(acc.items()):
        vals = list(per.values())
        print("| %s | %s | %d | %.1f |" % (name, ctr, len(vals), sum(vals) / len(vals)))


def _counter_means(path):
    """{kernel: mean KiB per dispatch} from a rocprofv3 counter_collection.csv (one counter)."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: (len(v), sum(v.values()) / len(v)) for k, v in acc.items()}


def counters(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same counters read for a
    plain device copy of T bytes each way, print a table, and write the dominant kernel's
    HBM bytes per launch to profiles/kl_bwd_pair8192_counters.json."""
    def one(d):
        return _counter_means(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0])

    fetch, write, cf, cw = one(fetch_dir), one(write_dir), one(cal_fetch_dir), one(cal_write_dir)
    copy_f = [v for k, v in cf.items() if "copyBuffer" in k][0][1]
    copy_w = [v for k, v in cw.items() if "copyBuffer" in k][0][1]
    kf, kw = T_BYTES / (copy_f * 1024.0), T_BYTES / (copy_w * 1024.0)
    print("Calibration: a device copy of %d bytes each way reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB "
          "per dispatch; scale factors %.5f (fetch) and %.5f (write)." % (T_BYTES, copy_f, copy_w, kf, kw))
    print()
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | in units of T |")
    print("|---|---|---|---|---|---|")
    dom = None
    for k in sorted(fetch):
        n, f = fetch[k]
        w = write.get(k, (0, 0.0))[1]
        bytes_ = f * 1024.0 * kf + w * 1024.0 * kw
        print("| %s | %d | %.1f | %.1f | %.0f | %.4f |" % (k, n, f, w, bytes_, bytes_ / T_BYTES))
        if k.startswith("void vws::bwd_kernel<2, 1, true"):
            dom = bytes_
    out = {"kernel": "bwd_kernel<KL,bf16,vec> on the 8192x75968 bf16 pair", "hbm_bytes_per_launch": round(dom),
           "fetch_factor": kf, "write_factor": kw, "kernel_source_hash": kernel_source_hash(),
           "sources": KERNEL_SOURCES}
    with open(os.path.join(PROFILE_DIR, "kl_bwd_pair8192_counters.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


# --------------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-linear", action="store_true", help="skip the fused linear-logp workload")
    ap.add_argument("--no-extras", action="store_true", help="skip top-k, JSD, fp16 and batch-invariant timings")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--summarize", nargs=2, metavar=("DIR", "MODE"))
    ap.add_argument("--counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"))
    args = ap.parse_args()

    if args.summarize:
        summarize(*args.summarize)
        return
    if args.counters:
        counters(*args.counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only; --gpus %d is not supported (rows would shard across GPUs with "
              "no communication, so the one-GPU figure is each GPU's share). Use --gpus 1." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    from vocab_wide_softmax_amd import workloads as W

    device = torch.device("cuda:0")
    if args.calibrate:
        calibrate(device)
        return

    log("generating the 8192x75968 bf16 pair on the host")
    wl = W.workload("pair8192")
    log("inputs ready")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_rows)
        log("cpu baseline: %s GB/s on %d threads" % (cpu["value"], cpu["cores"]))
    ms_per_step, med, dom_ms = gpu_bench(wl, args.steps, args.warmup, device)
    log("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step))
    value = STEP_BYTES / (ms_per_step * 1e-3) / 1e9
    achieved = DOMINANT_BYTES / (dom_ms * 1e-3) / 1e9
    ops = {}
    for op in ("logprobs", "entropy", "kl_ab", "kl_ba"):
        f, bw = med[op + "_fwd"], med[op + "_bwd"]
        ops[op] = {"fwd_ms": round(f, 4), "bwd_ms": round(bw, 4), "fwd_bwd_ms": round(f + bw, 4),
                   "GB/s": round(OP_BYTES[op] / ((f + bw) * 1e-3) / 1e9, 1),
                   "pct_peak": round(100 * OP_BYTES[op] / ((f + bw) * 1e-3) / 1e9 / PEAK_GBS, 1)}
    traffic = traffic_from_profiles()
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "8192x75968 bf16 logit pair (A~N(0,3^2), B=A+N(0,0.5^2), 5% rows +1e4, 1% rows "
                               "with 64 B columns at -inf); step = logprobs, entropy, KL(A||B), KL(B||A), each fwd+bwd",
                   "N": N_ROWS, "V": V, "step_bytes": STEP_BYTES},
        "pct_peak": round(100 * value / PEAK_GBS, 1),
        "ops": ops,
        "roofline": {"bound": "hbm", "kernel": "bwd_kernel<KL,bf16> (" + DOM_PHASE + ")", "achieved": round(achieved, 1),
                     "peak": PEAK_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": DOMINANT_BYTES,
                     "avg_launch_ms": round(dom_ms, 4)},
    }
    out["cpu_baseline"] = cpu
    if not args.no_extras:
        log("other ops: top-k logprobs, JSD, fp16 step, batch-invariant step")
        out["other_ops"] = extras_bench(wl, device)
    if not args.no_linear:
        out["linear_logp"] = linear_bench(max(3, args.steps // 4), 2, device)
        log("linear-logp: %.2f ms fwd, %.2f ms bwd" % (out["linear_logp"]["fwd_ms"], out["linear_logp"]["bwd_ms"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
