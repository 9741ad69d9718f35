"""Helpers for the GPU parity tests: run an op through the C ABI and compare with the fp64 oracle.

The device side goes through ``vocab_wide_softmax_amd.binding`` (ctypes over
libvws.so); the oracle side gets the same host tensors, upcast exactly to
float64. The two share nothing else.
"""

import numpy as np
import torch

from oracle import compare, reductions as R
from vocab_wide_softmax_amd import binding as B

OPS = ("logprobs", "entropy", "kl_ab", "kl_ba")
IGNORE = -100


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_device(op, a, b, t, g, split_hint=0, need_a=True, need_b=True):
    """Forward + backward of one op on the device; returns host float64 arrays."""
    if op == "logprobs":
        out, stats = B.logprobs_fwd(a, t, IGNORE, split_hint)
        grads = (B.logprobs_bwd(a, t, stats, g, IGNORE),)
    elif op == "entropy":
        out, stats = B.entropy_fwd(a, split_hint)
        grads = (B.entropy_bwd(a, stats, out, g),)
    else:
        x, y = (a, b) if op == "kl_ab" else (b, a)
        out, stats = B.kl_fwd(x, y, split_hint)
        grads = B.kl_bwd(x, y, stats, out, g, need_a=need_a, need_b=need_b)
    torch.cuda.synchronize()
    n = out.numel()
    res = {"out": f64(out).reshape(n), "stats": f64(stats)}
    res["grads"] = [None if d is None else f64(d).reshape(n, -1) for d in grads]
    return res


def run_oracle(op, a, b, t, g, chunk=128):
    """Oracle values, gradients and conditioning scales for rows of [n, V] float64 inputs."""
    n = a.shape[0]
    outs, stats, grads, c_out, c_grads = [], [], [], [], []
    for r0 in range(0, n, chunk):
        sl = slice(r0, min(n, r0 + chunk))
        A, Bm, T, G = a[sl], (b[sl] if b is not None else None), (t[sl] if t is not None else None), g[sl]
        if op == "logprobs":
            o, m, ls = R.logprobs_fwd(A, T, IGNORE)
            gr = [R.logprobs_bwd(A, T, G, IGNORE)]
            co = R.cond_logprobs_fwd(A, T, IGNORE)
            cg = [R.cond_logprobs_bwd(A, T, G, IGNORE)]
            st = np.stack([m, ls], axis=1)
        elif op == "entropy":
            o, m, ls = R.entropy_fwd(A)
            gr = [R.entropy_bwd(A, G)]
            co = R.cond_entropy_fwd(A)
            cg = [R.cond_entropy_bwd(A, G)]
            st = np.stack([m, ls], axis=1)
        else:
            X, Y = (A, Bm) if op == "kl_ab" else (Bm, A)
            o, (ma, lsa, mb, lsb) = R.kl_fwd(X, Y)
            gr = list(R.kl_bwd(X, Y, G))
            co = R.cond_kl_fwd(X, Y)
            cg = list(R.cond_kl_bwd(X, Y, G))
            st = np.stack([ma, lsa, mb, lsb], axis=1)
        outs.append(o)
        stats.append(st)
        grads.append(gr)
        c_out.append(co)
        c_grads.append(cg)
    k = len(grads[0])
    return {
        "out": np.concatenate(outs),
        "stats": np.concatenate(stats),
        "grads": [np.concatenate([gr[i] for gr in grads]) for i in range(k)],
        "c_out": np.concatenate(c_out),
        "c_grads": [np.concatenate([cg[i] for cg in c_grads]) for i in range(k)],
    }


def check_parity(dev, ora, grad_kind, label=""):
    """Assert the device results pass the acceptance rule of oracle.compare; returns the reports."""
    reports = {}
    r = compare.check(dev["out"], ora["out"], ora["c_out"], "f32")
    reports["out"] = r
    # statistics: the max is exact; log S within the fp32 rule, on defined rows
    st_d, st_o = dev["stats"], ora["stats"]
    for j in range(0, st_o.shape[1], 2):
        ok = np.isfinite(st_o[:, j])
        assert np.array_equal(st_d[ok, j], st_o[ok, j]), "%s: row max differs" % label
        rl = compare.check(st_d[ok, j + 1], st_o[ok, j + 1], np.abs(st_o[ok, j + 1]) + 1.0, "f32")
        reports["logS%d" % (j // 2)] = rl
    for i, (gd, go) in enumerate(zip(dev["grads"], ora["grads"])):
        if gd is None:
            continue
        reports["grad%d" % i] = compare.check(gd, go, ora["c_grads"][i], grad_kind)
    for name, rep in reports.items():
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, (label, name, rep)
    return reports
