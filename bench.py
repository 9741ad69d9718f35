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
bounded sample of the same workload on the host cores. Further legs, each in
its own object: the 1024 x 75968 pair (split-vocabulary path) with and without
a flush of the 256 MB Infinity Cache before every op, the fp32 causal-shift
view [4, 2049, 75968][:, :-1, :] read in place, extra peak device memory per op,
top-k logprobs, the JSD, fp16 and batch-invariant steps, and the fused
linear-logp with its own oracle baseline. The oracle leg also compares the
device results with the oracle on sampled rows of every workload and reports
the strict-rule misses per op and config.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --calibrate          # plain copies of known size, for counter scaling
    python bench.py --reference-rates    # torch's own streaming kernels at the headline size, as context
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


def extras_bench(wl, device, steps=15, warmup=60):
    """The other ops on the same 8192 x 75968 pair, each fwd+bwd, with their algorithmic bytes:
    top-k logprobs (K = 16 ids per row), the generalized JSD (beta = 0.5: two reads of both
    inputs forward, one read of both and two writes backward), the four-op step on fp16 copies
    of the logits, and the four-op step in the batch-invariant split mode. These legs start right
    after their inputs' host-to-device copies, when the card runs its first few dozen sub-ms
    kernels slower (top-k backward 0.47 ms there, 0.39 ms afterwards); each leg therefore warms
    up with 60 untimed calls before its 15 timed ones."""
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


# ------------------------------------------------------- per-op legs (configs 1 and 3)

def op_fwd(B, op, a, b, t, split=0):
    """Forward of one op through the C ABI: (per-row output, saved statistics)."""
    if op == "logprobs":
        return B.logprobs_fwd(a, t, -100, split)
    if op == "entropy":
        return B.entropy_fwd(a, split)
    x, y = (a, b) if op == "kl_ab" else (b, a)
    return B.kl_fwd(x, y, split)


def op_bwd(B, op, a, b, t, g, out, st):
    """Backward of one op: the tuple of gradients (two for KL)."""
    if op == "logprobs":
        return (B.logprobs_bwd(a, t, st, g, -100),)
    if op == "entropy":
        return (B.entropy_bwd(a, st, out, g),)
    x, y = (a, b) if op == "kl_ab" else (b, a)
    return B.kl_bwd(x, y, st, out, g)


def op_times(ops, a, b, t, g, steps, warmup, flush=None, split=0):
    """Median fwd and bwd ms per op, the ops interleaved (the pages interleave their timed runs).
    With `flush`, a device buffer of 512 MB is overwritten before every op's forward, outside the
    event interval, so that the op starts with nothing of its inputs in the 256 MB Infinity Cache
    or the L2 caches. `split` is the forwards' split_hint. All iterations are enqueued before one
    synchronisation."""
    import torch

    from vocab_wide_softmax_amd import binding as B

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for op in ops:
            out, st = op_fwd(B, op, a, b, t, split)
            op_bwd(B, op, a, b, t, g[op], out, st)
    evs = {op: [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)] for op in ops}
    torch.cuda.synchronize()
    for i in range(steps):
        for op in ops:
            if flush is not None:
                flush.zero_()
            e = evs[op][i]
            e[0].record(stream)
            out, st = op_fwd(B, op, a, b, t, split)
            e[1].record(stream)
            grads = op_bwd(B, op, a, b, t, g[op], out, st)
            e[2].record(stream)
            del out, st, grads
    torch.cuda.synchronize()
    res = {}
    for op in ops:
        f = sorted(e[0].elapsed_time(e[1]) for e in evs[op])
        bw = sorted(e[1].elapsed_time(e[2]) for e in evs[op])
        res[op] = (f[steps // 2], bw[steps // 2])
    return res


def _op_entry(f_ms, b_ms, nbytes):
    gbs = nbytes / ((f_ms + b_ms) * 1e-3) / 1e9
    return {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "fwd_bwd_ms": round(f_ms + b_ms, 4),
            "bytes": nbytes, "GB/s": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_GBS, 1)}


def memory_report(ops, a, b, t, g):
    """Device memory of one fwd+bwd per op, with the inputs already resident: the peak growth
    (torch.cuda.max_memory_allocated), the bytes of the gradients and of the per-row outputs and
    statistics the op returns, and the extra peak beyond those (workspace and anything else the
    op needs), which the pages report as "extra peak memory"."""
    import torch

    from vocab_wide_softmax_amd import binding as B

    rep = {}
    for op in ops:
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out, st = op_fwd(B, op, a, b, t)
        grads = op_bwd(B, op, a, b, t, g[op], out, st)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        grad_bytes = sum(x.numel() * x.element_size() for x in grads if x is not None)
        out_bytes = out.numel() * out.element_size() + st.numel() * st.element_size()
        rep[op] = {"peak_growth_bytes": int(peak), "grad_bytes": int(grad_bytes), "output_bytes": int(out_bytes),
                   "extra_peak_bytes": int(max(0, peak - grad_bytes - out_bytes)),
                   "workspace_bytes": int(B.workspace_bytes(B.OP_KL if op.startswith("kl") else
                                                            (B.OP_LOGPROBS if op == "logprobs" else B.OP_ENTROPY),
                                                            out.numel(), a.shape[-1]))}
        del out, st, grads
    return rep


def pair1024_leg(device, steps, warmup, wl=None):
    """The 1024 x 75968 bf16 pair (the shape of one of two tensor-parallel ranks of a 151936-token
    vocabulary): the four ops fwd+bwd, timed as they are (inputs of 156 MB each can sit in the
    256 MB Infinity Cache) and with the cache flushed before every op. The automatic launch does
    not split the vocabulary at 1024 rows (one workgroup per row already fills the chip; split
    forwards measured slower); `flushed_split8` times the forwards split into 8 parts merged by
    the in-GPU combine, the pages' cross-shard path, for comparison."""
    import torch

    from vocab_wide_softmax_amd import binding as B
    from vocab_wide_softmax_amd import workloads as W

    wl = wl or W.workload("pair1024")
    a, b, t = wl.a.to(device), wl.b.to(device), wl.t.to(device)
    g = {op: wl.g[op].to(device) for op in W.OPS}
    n, v = a.shape
    t1 = n * v * 2
    nbytes = {"logprobs": 3 * t1, "entropy": 3 * t1, "kl_ab": 6 * t1, "kl_ba": 6 * t1}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    warm = op_times(W.OPS, a, b, t, g, steps, warmup)
    cold = op_times(W.OPS, a, b, t, g, steps, warmup, flush=flush)
    cold8 = op_times(W.OPS, a, b, t, g, steps, warmup, flush=flush, split=8)
    out = {"workload": "1024x75968 bf16 pair (A~N(0,3^2), B=A+N(0,0.5^2), 5% rows +1e4, 1% rows with 64 B "
                       "columns at -inf)", "vocab_parts": B.split_parts(B.OP_KL, n, v),
           "unflushed": {}, "flushed": {}, "flushed_split8": {}}
    for op in W.OPS:
        out["unflushed"][op] = _op_entry(*warm[op], nbytes[op])
        out["flushed"][op] = _op_entry(*cold[op], nbytes[op])
        out["flushed_split8"][op] = _op_entry(*cold8[op], nbytes[op])
    for k, res in (("unflushed", warm), ("flushed", cold), ("flushed_split8", cold8)):
        tot = sum(sum(res[op]) for op in W.OPS)
        out[k]["all_four"] = _op_entry(tot, 0.0, sum(nbytes.values()))
    del flush
    torch.cuda.empty_cache()
    return out


def shifted_leg(device, steps, warmup, wl=None):
    """fp32 logits of two bases [4, 2049, 75968] read in place through the causal-shift
    view base[:, :-1, :] (8192 rows, two row strides, no copy): entropy(A) and KL(A||B) fwd+bwd
    (gradients fp32, contiguous), with the extra peak memory of each."""
    import torch

    from vocab_wide_softmax_amd import workloads as W

    wl = wl or W.workload("shifted")
    ab, bb, ib = wl.a_base.to(device), wl.b_base.to(device), wl.ids_base.to(device)
    a, b, t = wl.views(ab, bb, ib)
    assert not a.is_contiguous()
    g = {op: wl.g[op].to(device) for op in W.OPS}
    n = a.shape[0] * a.shape[1]
    t3 = n * a.shape[-1] * 4
    ops = ("entropy", "kl_ab")
    nbytes = {"entropy": 3 * t3, "kl_ab": 6 * t3}
    torch.cuda.synchronize()
    res = op_times(ops, a, b, t, g, steps, warmup)
    out = {"workload": "fp32 [4, 2049, 75968] pair ~ N(0, 3^2) read as base[:, :-1, :] (8192 rows, strides "
                       "2049x75968 and 75968 elements)", "ops": {op: _op_entry(*res[op], nbytes[op]) for op in ops},
           "memory": memory_report(ops, a, b, t, g)}
    del ab, bb, ib, a, b, t
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------- fused linear-logp

LIN_N, LIN_H, LIN_V = 8192, 4096, 151936
MFMA_BF16_PEAK_TFLOPS = 2500.0


def linear_bench(steps, warmup, device, wl=None):
    """Forward + backward of the fused linear-logp on h [8192, 4096], W [151936, 4096] bf16.
    Algorithmic FLOPs: forward 2 N H V; backward 3 x 2 N H V (logits recomputed, dh, dW). The
    backward feeds dz to the dh and dW contractions as a bf16 (hi, lo) pair, so the MFMA work it
    executes is 5 x 2 N H V; both rates are reported."""
    import torch

    from vocab_wide_softmax_amd import binding as B
    from vocab_wide_softmax_amd import workloads as W

    wl = wl or W.linear_logp(LIN_N, LIN_H, LIN_V)
    h, Wm, t, g = wl.h.to(device), wl.W.to(device), wl.t.to(device), wl.g.to(device)
    n, hidden = h.shape
    v = Wm.shape[0]
    ws_bytes = B.linear_workspace_bytes(1, n, hidden, v)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    torch.cuda.synchronize()
    log("linear-logp inputs resident; %d warmup steps" % warmup)
    for _ in range(warmup):
        lp, st = B.linear_logp_fwd(h, Wm, t)
        B.linear_logp_bwd(h, Wm, t, st, g, ws=ws)
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        lp, st = B.linear_logp_fwd(h, Wm, t)
        evs[i][1].record(stream)
        B.linear_logp_bwd(h, Wm, t, st, g, ws=ws)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    fwd = sorted(e[0].elapsed_time(e[1]) for e in evs)[steps // 2]
    bwd = sorted(e[1].elapsed_time(e[2]) for e in evs)[steps // 2]
    flop = 2.0 * n * hidden * v
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12
    del ws
    torch.cuda.empty_cache()
    return {
        "workload": "h [8192, 4096] ~ N(0,1), W [151936, 4096] ~ N(0, 0.02^2), bf16; targets U[0, 151936)",
        "ms_per_step": round(wall, 3), "fwd_ms": round(fwd, 3), "bwd_ms": round(bwd, 3),
        "fwd_tflops": round(tf(flop, fwd), 1), "bwd_tflops": round(tf(3 * flop, bwd), 1),
        "step_tflops": round(tf(4 * flop, fwd + bwd), 1),
        "bwd_workspace_bytes": int(ws_bytes),
        "roofline": {"bound": "mfma", "achieved": round(tf(4 * flop, fwd + bwd), 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf(4 * flop, fwd + bwd) / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_step": 4 * flop,
                     "executed_mfma_flop_per_step": 6 * flop,
                     "executed_frac": round(tf(6 * flop, fwd + bwd) / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


def library_gemm(device, wl=None, reps=5):
    """Context for the fused linear-logp's roofline, not part of the path: torch's own bf16 GEMM
    (hipBLASLt) on the products the path computes, at the same shapes and on the same h and W (dz
    random, N(0, 1e-8)), timed with HIP events on torch's stream: the full logits h W^T, one
    8192-column chunk of them, and the chunk's dW = dz^T h and dh = dz W_chunk with a single bf16
    dz (the path contracts a hi + lo pair, twice that work)."""
    import torch

    from vocab_wide_softmax_amd import workloads as W

    wl = wl or W.linear_logp(LIN_N, LIN_H, LIN_V)
    h, Wm = wl.h.to(device), wl.W.to(device)
    n, hidden = h.shape
    v, c = Wm.shape[0], 8192
    wc = Wm[:c].contiguous()
    gen = torch.Generator().manual_seed(11)
    dz = (torch.randn(n, c, generator=gen) * 1e-4).to(torch.bfloat16).to(device)
    cases = (("logits_h_Wt_8192x151936x4096", lambda: h @ Wm.t(), 2.0 * n * v * hidden),
             ("chunk_logits_h_Wct_8192x8192x4096", lambda: h @ wc.t(), 2.0 * n * c * hidden),
             ("chunk_dW_dzt_h_8192x4096x8192", lambda: dz.t() @ h, 2.0 * c * hidden * n),
             ("chunk_dh_dz_Wc_8192x4096x8192", lambda: dz @ wc, 2.0 * n * hidden * c))
    out = {}
    stream = torch.cuda.current_stream()
    for name, f, flop in cases:
        for _ in range(2):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 3), "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1)}
    del h, Wm, wc, dz
    torch.cuda.empty_cache()
    return out


def linear_cpu_baseline(wl, rows=512, vocab_rows=512):
    """The fp64 oracle of the fused linear-logp on a sub-batch of `rows` evenly spaced tokens of
    the same workload: logp (forward over the full vocabulary), dh of those tokens, and the rows of
    dW for `vocab_rows` vocabulary entries (targeted and untargeted) summed over that sub-batch.
    TFLOP/s counts the algorithmic work of those outputs (forward 2 n H V, logits recomputed
    2 n H V, dh 2 n V H, dW rows 2 n r H); BLAS runs on the host's threads."""
    import numpy as np

    from oracle import linear_logp as OL

    n_all, hidden = wl.h.shape
    v = wl.W.shape[0]
    idx = np.linspace(0, n_all - 1, rows).astype(np.int64)
    h = wl.h[idx].double().numpy()
    W = wl.W.double().numpy()
    t = wl.t[idx].numpy()
    g = wl.g[idx].double().numpy()
    rng = np.random.default_rng(7)
    cols = np.unique(np.concatenate([t[: vocab_rows // 4], rng.choice(v, vocab_rows, replace=False)]))[:vocab_rows]
    t0 = time.perf_counter()
    OL.linear_logp_fwd(h, W, t)
    OL.linear_logp_bwd_dh(h, W, t, g)
    OL.linear_logp_bwd_dw(h, W, t, g, vocab_rows=cols)
    el = time.perf_counter() - t0
    flop = 3 * 2.0 * rows * hidden * v + 2.0 * rows * len(cols) * hidden
    return {"value": round(flop / el / 1e12, 4), "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": "%d of %d tokens (evenly spaced) of h [8192, 4096] x W [151936, 4096]: float64 logp over the "
                      "full vocabulary, dh of those tokens, and %d rows of dW (a quarter of them targeted) summed "
                      "over them; %.1f s wall; TFLOP/s = algorithmic FLOPs of those outputs / wall time"
                      % (rows, n_all, len(cols), el)}


def _blas_threads():
    """Threads of the host BLAS that the oracle's matrix products run on."""
    try:
        from threadpoolctl import threadpool_info

        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


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

    cores = len(os.sched_getaffinity(0))
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


def _sample(wl, n, k, seed=5):
    """Rows to compare: first and last, offset and masked rows of the recipe, and k random rows."""
    import numpy as np

    rng = np.random.default_rng(seed)
    rows = {0, n - 1}
    rows.update(wl.offset_rows[:4].tolist())
    rows.update(wl.mask_rows[:4].tolist())
    rows.update(rng.choice(n, size=min(k, n), replace=False).tolist())
    return np.array(sorted(rows))


def _rep(x, y, c, kind):
    from oracle import compare

    r = compare.check(x, y, c, kind)
    return {k: (float("%.3g" % v) if k == "max_rel" else round(v, 4)) if isinstance(v, float) else v
            for k, v in r.items()}


def _oracle_op(op, a, b, t, g):
    """(output, gradients, output scale, gradient scales) of the oracle for float64 rows."""
    from oracle import reductions as R

    if op == "logprobs":
        return (R.logprobs_fwd(a, t)[0], [R.logprobs_bwd(a, t, g)], R.cond_logprobs_fwd(a, t),
                [R.cond_logprobs_bwd(a, t, g)])
    if op == "entropy":
        return R.entropy_fwd(a)[0], [R.entropy_bwd(a, g)], R.cond_entropy_fwd(a), [R.cond_entropy_bwd(a, g)]
    x, y = (a, b) if op == "kl_ab" else (b, a)
    return R.kl_fwd(x, y)[0], list(R.kl_bwd(x, y, g)), R.cond_kl_fwd(x, y), list(R.cond_kl_bwd(x, y, g))


def oracle_parity(device, wls, lin_wl, with_dw=True):
    """Part of the oracle leg: the device results of each workload's launch (the configuration the
    bench times) against the fp64 oracle on sampled rows, under the acceptance rule of
    oracle/compare.py. Per config and op: elements compared, strict-rule misses, failures of both
    rules (must be 0), NaN / inf placement mismatches and the worst error-to-allowance ratio."""
    import numpy as np
    import torch

    from oracle import linear_logp as OL
    from vocab_wide_softmax_amd import binding as B
    from vocab_wide_softmax_amd import workloads as W

    out = {}
    cases = (("tiny_64x1024_fp32", "tiny", W.OPS, "f32", None, 0),
             ("tiny_64x1024_fp32_split16", "tiny", W.OPS, "f32", None, 16),
             ("pair_1024x75968_bf16", "pair1024", W.OPS, "bf16", 24, 0),
             ("pair_8192x75968_bf16", "pair8192", W.OPS, "bf16", 24, 0),
             ("shifted_fp32_4x2049x75968", "shifted", ("entropy", "kl_ab"), "f32", 12, 0))
    for label, key, ops, kind, k, split in cases:
        wl = wls[key]
        if wl.shifted:
            a, b, t = wl.views(wl.a_base.to(device), wl.b_base.to(device), wl.ids_base.to(device))
        else:
            a, b, t = wl.a.to(device), wl.b.to(device), wl.t.to(device)
        V = a.shape[-1]
        n = a.numel() // V
        rows = np.arange(n) if k is None else _sample(wl, n, k)
        idx = torch.from_numpy(rows).to(device)
        if wl.shifted:  # host rows of the causal-shift view without materialising it
            s_in = wl.a_base.shape[1] - 1
            pick = lambda base: torch.stack([base[r // s_in, r % s_in] for r in rows.tolist()]).double().numpy()
            ha, hb = pick(wl.a_base), pick(wl.b_base)
            ht = torch.stack([wl.ids_base[r // s_in, r % s_in + 1] for r in rows.tolist()]).numpy()
        else:
            ha, hb, ht = wl.a[rows].double().numpy(), wl.b[rows].double().numpy(), wl.t[rows].numpy()
        res = {}
        for op in ops:
            gd = wl.g[op].to(device)
            o, st = op_fwd(B, op, a, b, t, split)
            grads = op_bwd(B, op, a, b, t, gd, o, st)
            do = o.reshape(-1)[idx].double().cpu().numpy()
            dg = [x.reshape(-1, V)[idx].double().cpu().numpy() for x in grads]
            del o, st, grads
            yo, yg, co, cg = _oracle_op(op, ha, hb, ht, wl.g[op][rows].double().numpy())
            r = {"out": _rep(do, yo, co, "f32")}
            names = ["grad"] if len(yg) == 1 else (["grad_a", "grad_b"] if op == "kl_ab" else ["grad_b", "grad_a"])
            for nm, x, y, c in zip(names, dg, yg, cg):
                r[nm] = _rep(x, y, c, kind)
            res[op] = r
        res["rows_compared"] = int(len(rows))
        out[label] = res
        del a, b, t
        torch.cuda.empty_cache()
        log("parity %s done" % label)
    # the fused linear-logp (8192 x 4096 x 151936) in the benchmark's launch
    h, Wm, t, g = lin_wl.h.to(device), lin_wl.W.to(device), lin_wl.t.to(device), lin_wl.g.to(device)
    lp, st = B.linear_logp_fwd(h, Wm, t)
    dh, dW = B.linear_logp_bwd(h, Wm, t, st, g)
    hh, hw, ht, hg = (lin_wl.h.double().numpy(), lin_wl.W.double().numpy(), lin_wl.t.numpy(),
                      lin_wl.g.double().numpy())
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, hh.shape[0] - 1], rng.integers(0, hh.shape[0], 14)]))
    idx = torch.from_numpy(rows).to(device)
    r = {"logp": _rep(lp[idx].double().cpu().numpy(), OL.linear_logp_fwd(hh, hw, ht, rows=rows)[0],
                      OL.cond_linear_fwd(hh, hw, ht, rows=rows), "f32"),
         "dh": _rep(dh[idx].double().cpu().numpy(), OL.linear_logp_bwd_dh(hh, hw, ht, hg, rows=rows),
                    OL.cond_linear_dh(hh, hw, ht, hg, rows=rows), "bf16"),
         "rows_compared": int(len(rows))}
    if with_dw:
        untargeted = np.setdiff1d(np.arange(hw.shape[0]), ht)
        cols = np.unique(np.concatenate([ht[:16], rng.choice(untargeted, 48, replace=False)]))
        ref, c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg, vocab_rows=cols)
        r["dW"] = _rep(dW[torch.from_numpy(cols).to(device)].double().cpu().numpy(), ref, c, "bf16")
        r["dW_vocab_rows_compared"] = int(len(cols))
    out["linear_logp_8192x4096x151936_bf16"] = r
    del h, Wm, t, g, lp, st, dh, dW
    torch.cuda.empty_cache()
    return out


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


def reference_rates(device, reps=20):
    """HBM rates of torch's own streaming kernels on one bf16 [8192, 75968] tensor (T bytes), as
    context for the roofline fractions: an elementwise multiply (read T, write T), a device copy
    (hipMemcpy, read T, write T), a fill (write T) and an elementwise multiply of two tensors (read
    2 T, write T). Medians of `reps` launches timed with HIP events."""
    import torch

    n = T_BYTES // 2
    a = torch.empty(n, dtype=torch.bfloat16, device=device).normal_()
    b = torch.empty_like(a).normal_()
    c = torch.empty_like(a)
    torch.cuda.synchronize()

    def med(fn):
        for _ in range(5):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        s = torch.cuda.current_stream()
        for x, y in ev:
            x.record(s)
            fn()
            y.record(s)
        torch.cuda.synchronize()
        return sorted(x.elapsed_time(y) for x, y in ev)[reps // 2]

    out = {}
    for name, fn, nbytes in (("mul_scalar_read_write", lambda: torch.mul(a, 2.0, out=c), 2 * T_BYTES),
                             ("device_copy_read_write", lambda: c.copy_(a), 2 * T_BYTES),
                             ("fill_write", lambda: c.fill_(1.0), T_BYTES),
                             ("mul_two_inputs_read2_write1", lambda: torch.mul(a, b, out=c), 3 * T_BYTES)):
        ms = med(fn)
        out[name] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_GBS, 1)}
    print(json.dumps({"reference_rates_bf16_8192x75968": out}))


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
    mode "counters": mean value per dispatch of every collected counter, per kernel;
    mode "gemm": clock, MFMA-busy and wait fractions of the MFMA kernels (see _summarize_gemm).
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
    if mode == "gemm":
        _summarize_gemm(con)
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


def _summarize_gemm(con, cus=256, xcds=8):
    """Per MFMA kernel (the linear-logp GEMMs and torch's Cijk GEMMs), from one counter run of
    GRBM_GUI_ACTIVE, SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT and SQ_BUSY_CYCLES: GRBM_GUI_ACTIVE sums the XCDs, so
    cycles = value / xcds; clock = cycles / kernel duration; MFMA busy = MFMA busy cycles / (4 cus
    SIMDs x cycles); waves per SIMD = SQ_WAVE_CYCLES (quad-cycles) x 4 / (4 cus x cycles); wait and
    issue-wait fractions = SQ_WAIT_ANY and SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES (all quad-cycles);
    LDS index active = SQ_LDS_IDX_ACTIVE / (cus x cycles)."""
    rows = con.execute("select dispatch_id, kernel_name, counter_name, sum(value), avg(duration) "
                       "from counters_collection group by dispatch_id, counter_name").fetchall()
    per = {}
    for did, kn, cn, v, dur in rows:
        e = per.setdefault(did, {"name": kn, "dur": dur})
        e[cn] = v
    groups = {}
    for e in per.values():
        n = e["name"]
        if "lin_" in n and ("fwd_kernel" in n or "dz_kernel" in n) or "gemm_pair" in n or "Cijk" in n:
            groups.setdefault(n, []).append(e)
    print("| kernel | dispatches | mean us | clock GHz | MFMA busy | waves / SIMD | wait | issue wait "
          "| LDS index active | LDS bank conflicts / dispatch |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for n, es in sorted(groups.items(), key=lambda kv: -sum(e["dur"] for e in kv[1])):
        m = {k: sum(e.get(k, 0.0) for e in es) / len(es) for k in es[0] if k != "name"}
        cyc = m["GRBM_GUI_ACTIVE"] / xcds
        wc = max(m.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        label = n if len(n) < 110 else n[:60] + "..." + n[-40:]
        print("| %s | %d | %.1f | %.2f | %.1f%% | %.2f | %.2f | %.2f | %.1f%% | %.0f |" % (
            label, len(es), m["dur"] / 1e3, cyc / m["dur"],
            100 * m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * cus * cyc), 4 * wc / (4 * cus * cyc),
            m.get("SQ_WAIT_ANY", 0.0) / wc, m.get("SQ_WAIT_INST_ANY", 0.0) / wc,
            100 * m.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cus * cyc), m.get("SQ_LDS_BANK_CONFLICT", 0.0)))


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


def _raw_counter_sums(d):
    """{kernel: {counter: mean per dispatch}} from a rocprofv3 counter_collection.csv holding
    several raw counters (instances summed per dispatch)."""
    path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            k = acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})
            k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {kern: {c: sum(v.values()) / len(v) for c, v in cs.items()} for kern, cs in acc.items()}


def _read_bytes(c):
    """Read bytes from the request counts by size: 32-, 64- and 128-byte requests."""
    rd, r32, r128 = c.get("TCC_EA0_RDREQ", 0.0), c.get("TCC_EA0_RDREQ_32B", 0.0), c.get("TCC_EA0_RDREQ_128B", 0.0)
    return r32 * 32 + r128 * 128 + (rd - r32 - r128) * 64


def _fetch_size_formula_bytes(c):
    """The stock FETCH_SIZE expression (in bytes): 128-byte requests counted through TCC_BUBBLE."""
    rd, r32, bub = c.get("TCC_EA0_RDREQ", 0.0), c.get("TCC_EA0_RDREQ_32B", 0.0), c.get("TCC_BUBBLE", 0.0)
    return bub * 128 + (rd - bub - r32) * 64 + r32 * 32


def _write_bytes(c):
    wr, w64 = c.get("TCC_EA0_WRREQ", 0.0), c.get("TCC_EA0_WRREQ_64B", 0.0)
    return (wr - w64) * 32 + w64 * 64


def counters_raw(rd_dir, wr_dir, cal_rd_dir, cal_wr_dir):
    """HBM bytes per kernel from the L2-to-memory request counts by request size (no fitted factor):
    reads = 32 B x RDREQ_32B + 128 B x RDREQ_128B + 64 B x the rest of RDREQ, writes =
    32 B x (WRREQ - WRREQ_64B) + 64 B x WRREQ_64B. The plain device copy of T bytes each way checks
    the derivation against known traffic; the stock FETCH_SIZE expression, which counts 128-byte
    requests through TCC_BUBBLE, is shown beside it. Writes the dominant kernel's bytes per launch
    to profiles/kl_bwd_pair8192_counters.json."""
    rd, wr, crd, cwr = (_raw_counter_sums(x) for x in (rd_dir, wr_dir, cal_rd_dir, cal_wr_dir))
    copy = [k for k in crd if "copyBuffer" in k or "copy" in k.lower()][0]
    cr, cw = _read_bytes(crd[copy]), _write_bytes(cwr[copy])
    print("Calibration copy (%d bytes each way): request-size reads %.0f bytes (ratio %.5f), writes %.0f bytes "
          "(ratio %.5f); the stock FETCH_SIZE expression gives %.0f bytes (ratio %.5f): RDREQ %.0f, 32B %.0f, "
          "128B %.0f, BUBBLE %.0f." % (T_BYTES, cr, cr / T_BYTES, cw, cw / T_BYTES, _fetch_size_formula_bytes(crd[copy]),
                                      _fetch_size_formula_bytes(crd[copy]) / T_BYTES, crd[copy].get("TCC_EA0_RDREQ", 0),
                                      crd[copy].get("TCC_EA0_RDREQ_32B", 0), crd[copy].get("TCC_EA0_RDREQ_128B", 0),
                                      crd[copy].get("TCC_BUBBLE", 0)))
    print()
    print("| kernel | RDREQ | RDREQ_32B | RDREQ_128B | BUBBLE | WRREQ | WRREQ_64B | read bytes | write bytes | "
          "total / T | FETCH_SIZE expression bytes |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    dom = None
    for k in sorted(rd):
        c, w = rd[k], wr.get(k, {})
        rb, wb = _read_bytes(c), _write_bytes(w)
        print("| %s | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.4f | %.0f |" % (
            k, c.get("TCC_EA0_RDREQ", 0), c.get("TCC_EA0_RDREQ_32B", 0), c.get("TCC_EA0_RDREQ_128B", 0),
            c.get("TCC_BUBBLE", 0), w.get("TCC_EA0_WRREQ", 0), w.get("TCC_EA0_WRREQ_64B", 0), rb, wb,
            (rb + wb) / T_BYTES, _fetch_size_formula_bytes(c)))
        if k.startswith("void vws::bwd_kernel<2, 1, true"):
            dom = rb + wb
    out = {"kernel": "bwd_kernel<KL,bf16,vec> on the 8192x75968 bf16 pair", "hbm_bytes_per_launch": round(dom),
           "method": "L2-to-memory request counts by size (TCC_EA0_RDREQ, _32B, _128B; TCC_EA0_WRREQ, _64B), "
                     "no fitted factor", "calibration_copy_ratio": {"read": cr / T_BYTES, "write": cw / T_BYTES},
           "kernel_source_hash": kernel_source_hash(), "sources": KERNEL_SOURCES}
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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 1024x75968 (flushed / unflushed) and fp32 causal-shift legs")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle comparison on sampled rows")
    ap.add_argument("--parity-no-dw", action="store_true",
                    help="in the oracle comparison, skip the dW rows of the fused linear-logp (full-batch fp64 logits)")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--cpu-linear-rows", type=int, default=512)
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch's bf16 GEMM (hipBLASLt) on the linear-logp products, as context")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--reference-rates", action="store_true",
                    help="only time torch's own streaming kernels on the headline tensor size, as context")
    ap.add_argument("--summarize", nargs=2, metavar=("DIR", "MODE"))
    ap.add_argument("--counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"))
    ap.add_argument("--counters-raw", nargs=4, metavar=("RD_DIR", "WR_DIR", "CAL_RD_DIR", "CAL_WR_DIR"),
                    help="HBM bytes from request counts by size (TCC_EA0_RDREQ/_32B/_128B, TCC_BUBBLE; "
                         "TCC_EA0_WRREQ/_64B)")
    args = ap.parse_args()

    if args.summarize:
        summarize(*args.summarize)
        return
    if args.counters:
        counters(*args.counters)
        return
    if args.counters_raw:
        counters_raw(*args.counters_raw)
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
    if args.reference_rates:
        reference_rates(device)
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
    # extra peak device memory of each op at the headline shape (inputs resident)
    _, a, b, t, g = make_inputs(wl, device)
    out["memory"] = memory_report(W.OPS, a, b, t, g)
    del a, b, t, g
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("other ops: top-k logprobs, JSD, fp16 step, batch-invariant step")
        out["other_ops"] = extras_bench(wl, device)
    wl1024 = wl_shift = None
    if not args.no_configs:
        log("1024x75968 pair: unflushed and flushed")
        wl1024 = W.workload("pair1024")
        out["pair1024"] = pair1024_leg(device, args.steps, 5, wl1024)
        log("fp32 causal-shift view [4, 2049, 75968][:, :-1]")
        wl_shift = W.workload("shifted")
        out["shifted_fp32"] = shifted_leg(device, max(5, args.steps // 2), 3, wl_shift)
    lin_wl = None
    if not args.no_linear:
        lin_wl = W.linear_logp(LIN_N, LIN_H, LIN_V)
        out["linear_logp"] = linear_bench(max(3, args.steps // 4), 2, device, lin_wl)
        log("linear-logp: %.2f ms fwd, %.2f ms bwd" % (out["linear_logp"]["fwd_ms"], out["linear_logp"]["bwd_ms"]))
        if args.library_gemm:
            out["linear_logp"]["library_gemm"] = library_gemm(device, lin_wl)
            log("library GEMM reference: %s" % json.dumps(out["linear_logp"]["library_gemm"]))
        if not args.no_cpu_baseline:
            out["linear_logp"]["cpu_baseline"] = linear_cpu_baseline(lin_wl, args.cpu_linear_rows)
            log("linear-logp cpu baseline: %s TFLOP/s" % out["linear_logp"]["cpu_baseline"]["value"])
    if not args.no_cpu_baseline and not args.no_parity:
        # the oracle leg's comparison of device results with the oracle on sampled rows
        wls = {"tiny": W.workload("tiny"), "pair8192": wl, "pair1024": wl1024 or W.workload("pair1024"),
               "shifted": wl_shift or W.workload("shifted")}
        lin_wl = lin_wl or W.linear_logp(LIN_N, LIN_H, LIN_V)
        out["parity"] = oracle_parity(device, wls, lin_wl, with_dw=not args.parity_no_dw)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
