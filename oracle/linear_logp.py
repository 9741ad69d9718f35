"""fp64 definition of the fused linear-logp op (test infrastructure only).

Source: RL-Kernel PR #208 "[Feat][Kernel] Add TP Fused linear logp Triton"
(PR body, "Implementation"): the logits z = h W^T are never materialised by
the kernel; the forward returns, per row, the log-probability of the target
token and the log-sum-exp, logp = z_t - lse. The backward (the chunked
PyTorch backward named in the PR and in the review nitpick) forms
dz = g (onehot(t) - softmax(z)) and then dh = dz W, dW = dz^T h by the chain
rule.

Here z is formed in float64 by a plain matrix product and handed to the
per-row definitions in ``oracle.reductions``. Row blocks (``rows`` argument or
``row_chunk``) only bound memory: rows are independent, so evaluating a subset
of rows changes no arithmetic.
"""

import numpy as np

from . import reductions

__all__ = ["logits", "linear_logp_fwd", "linear_logp_bwd_dz", "linear_logp_bwd_dh", "linear_logp_bwd_dw",
           "cond_logits", "cond_linear_fwd", "cond_linear_dz", "cond_linear_dh", "cond_linear_dw",
           "linear_logp_bwd_dw_cond"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def logits(h, W, rows=None):
    """z = h W^T in float64 for the selected rows (all rows when rows is None)."""
    h = _f64(h)
    W = _f64(W)
    if rows is not None:
        h = h[np.asarray(rows)]
    return h @ W.T


def cond_logits(h, W, rows=None):
    """sum_k |h_nk W_vk|: the magnitude sum behind each logit."""
    h = np.abs(_f64(h))
    W = np.abs(_f64(W))
    if rows is not None:
        h = h[np.asarray(rows)]
    return h @ W.T


def linear_logp_fwd(h, W, t, ignore_index=-100, rows=None):
    """(logp [r], m [r], logS [r]) for the selected rows; lse = m + logS."""
    t = np.asarray(t, dtype=np.int64)
    if rows is not None:
        t = t[np.asarray(rows)]
    z = logits(h, W, rows)
    return reductions.logprobs_fwd(z, t, ignore_index)


def linear_logp_bwd_dz(h, W, t, g, ignore_index=-100, rows=None):
    """dz = g (onehot(t) - p) of the selected rows: the gradient of g logp with respect to the logits."""
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    if rows is not None:
        t = t[np.asarray(rows)]
        g = g[np.asarray(rows)]
    return reductions.logprobs_bwd(logits(h, W, rows), t, g, ignore_index)


def linear_logp_bwd_dh(h, W, t, g, ignore_index=-100, rows=None):
    """dh = dz W for the selected rows, dz = g (onehot(t) - p)."""
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    if rows is not None:
        t = t[np.asarray(rows)]
        g = g[np.asarray(rows)]
    z = logits(h, W, rows)
    dz = reductions.logprobs_bwd(z, t, g, ignore_index)
    return dz @ _f64(W)


def linear_logp_bwd_dw(h, W, t, g, ignore_index=-100, vocab_rows=None, row_chunk=512):
    """dW = dz^T h for the selected vocabulary rows (all when None).

    Needs every row's softmax, so z is formed block by block over the token
    rows (row_chunk at a time) and only the requested vocabulary columns of dz
    are kept.
    """
    h = _f64(h)
    W = _f64(W)
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    n = h.shape[0]
    cols = np.arange(W.shape[0]) if vocab_rows is None else np.asarray(vocab_rows)
    dW = np.zeros((len(cols), h.shape[1]))
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        z = h[r0:r1] @ W.T
        dz = reductions.logprobs_bwd(z, t[r0:r1], g[r0:r1], ignore_index)
        dW += dz[:, cols].T @ h[r0:r1]
    return dW


# Conditioning scales (sums of magnitudes of the terms each result combines),
# used by the parity rule. The logits themselves are sums over the hidden dim,
# so their magnitude sums |h| |W|^T enter every result built from them.

def cond_linear_fwd(h, W, t, ignore_index=-100, rows=None):
    """|z_t - m| + |log S| + cz_t + sum_v p_v cz_v, with cz = |h| |W|^T."""
    t = np.asarray(t, dtype=np.int64)
    if rows is not None:
        t = t[np.asarray(rows)]
    z = logits(h, W, rows)
    cz = cond_logits(h, W, rows)
    n, V = z.shape
    lp, m, logS = reductions.log_softmax_rows(z)
    p = np.exp(lp)
    c = np.abs(logS) + np.sum(p * cz, axis=1)
    ok = (t >= 0) & (t < V) & (t != ignore_index)
    r = np.nonzero(ok)[0]
    c[r] += np.abs(z[r, t[r]] - m[r]) + cz[r, t[r]]
    return c


def cond_linear_dz(h, W, t, g, ignore_index=-100, rows=None):
    """Scale of dz_nv: the logits-op scale |g| (1[v = t] + p_v (1 + |z_v - m| + |log S|)) plus
    |g| p_v (cz_v + sum_u p_u cz_u), the rounding of the logit itself and of log S behind it."""
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    if rows is not None:
        t = t[np.asarray(rows)]
        g = g[np.asarray(rows)]
    z = logits(h, W, rows)
    cz = cond_logits(h, W, rows)
    p = np.exp(reductions.log_softmax_rows(z)[0])
    c = reductions.cond_logprobs_bwd(z, t, g, ignore_index)
    extra = np.abs(g)[:, None] * p * (cz + np.sum(p * cz, axis=1, keepdims=True))
    live = (t != ignore_index)[:, None]
    return c + np.where(live, extra, 0.0)


def cond_linear_dh(h, W, t, g, ignore_index=-100, rows=None):
    """sum_v |dz_nv| |W_vk|."""
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    if rows is not None:
        t = t[np.asarray(rows)]
        g = g[np.asarray(rows)]
    dz = reductions.logprobs_bwd(logits(h, W, rows), t, g, ignore_index)
    return np.abs(dz) @ np.abs(_f64(W))


def cond_linear_dw(h, W, t, g, ignore_index=-100, vocab_rows=None, row_chunk=512):
    """sum_n |dz_nv| |h_nk| for the selected vocabulary rows."""
    h = _f64(h)
    W = _f64(W)
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    cols = np.arange(W.shape[0]) if vocab_rows is None else np.asarray(vocab_rows)
    c = np.zeros((len(cols), h.shape[1]))
    for r0 in range(0, h.shape[0], row_chunk):
        r1 = min(h.shape[0], r0 + row_chunk)
        dz = reductions.logprobs_bwd(h[r0:r1] @ W.T, t[r0:r1], g[r0:r1], ignore_index)
        c += np.abs(dz[:, cols]).T @ np.abs(h[r0:r1])
    return c


def linear_logp_bwd_dw_cond(h, W, t, g, ignore_index=-100, vocab_rows=None, row_chunk=512):
    """(dW, its conditioning scale) for the selected vocabulary rows in one pass over the token rows."""
    h = _f64(h)
    W = _f64(W)
    t = np.asarray(t, dtype=np.int64)
    g = _f64(g).reshape(-1)
    cols = np.arange(W.shape[0]) if vocab_rows is None else np.asarray(vocab_rows)
    dW = np.zeros((len(cols), h.shape[1]))
    c = np.zeros_like(dW)
    for r0 in range(0, h.shape[0], row_chunk):
        r1 = min(h.shape[0], r0 + row_chunk)
        dz = reductions.logprobs_bwd(h[r0:r1] @ W.T, t[r0:r1], g[r0:r1], ignore_index)[:, cols]
        dW += dz.T @ h[r0:r1]
        c += np.abs(dz).T @ np.abs(h[r0:r1])
    return dW, c
