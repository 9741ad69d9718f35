"""fp64 definition of multi-id (top-k) log-probabilities (test infrastructure only).

Source: DeepSpeed PR #8838 "Add Triton kernels for vocab-parallel logprobs,
entropy and KL" -- the logprobs cases in the PR description's test list include
repeated ids, ignored ids and rows whose ids are all ignored, so the logprobs op
takes K ids per row.

Reading taken (the pages list the cases, not the values):

* ids has shape [n, K]; out[n, k] = log p_n(ids[n, k]) with the row's
  log-softmax (the single-id definition of ``reductions.logprobs_fwd`` applied
  to each slot);
* a slot equal to ``ignore_index`` gives 0 and adds nothing to the gradient;
* a slot outside [0, V) that is not ignored gives NaN, and the row's gradient
  is NaN (no status without a host synchronisation);
* the gradient of sum_k g[n, k] out[n, k] is
      dz_j = sum_{k live, ids[n, k] = j} g[n, k] - (sum_{k live} g[n, k]) p_j,
  so duplicate ids add their upstream gradients; a row whose slots are all
  ignored has an all-zero gradient, whatever its logits;
* an undefined row (NaN, +inf, or no entry above -inf) gives NaN at every
  live slot and a NaN gradient row unless all its slots are ignored.

Evaluated in float64 from the row's log-softmax, one slot at a time.
"""

import numpy as np

from .reductions import log_softmax_rows

__all__ = [
    "logprobs_topk_fwd",
    "logprobs_topk_bwd",
    "cond_logprobs_topk_fwd",
    "cond_logprobs_topk_bwd",
]

_ERR = dict(invalid="ignore", over="ignore", divide="ignore", under="ignore")


def _slots(ids, V, ignore_index):
    ids = np.asarray(ids, dtype=np.int64)
    ignored = ids == ignore_index
    bad = ~ignored & ((ids < 0) | (ids >= V))
    live = ~ignored & ~bad
    return ids, ignored, bad, live


def logprobs_topk_fwd(z, ids, ignore_index=-100):
    """out[n, k] = log p_n(ids[n, k]); returns (out [n, K], m [n], logS [n])."""
    z = np.asarray(z, dtype=np.float64)
    n, V = z.shape
    lp, m, logS = log_softmax_rows(z)
    ids, ignored, bad, live = _slots(ids, V, ignore_index)
    K = ids.shape[1]
    out = np.empty((n, K))
    for r in range(n):
        for k in range(K):
            if ignored[r, k]:
                out[r, k] = 0.0
            elif bad[r, k]:
                out[r, k] = np.nan
            else:
                out[r, k] = lp[r, ids[r, k]]
    return out, m, logS


def logprobs_topk_bwd(z, ids, g, ignore_index=-100):
    """Gradient of sum_k g[n, k] out[n, k] with respect to z (see the module text)."""
    z = np.asarray(z, dtype=np.float64)
    n, V = z.shape
    g = np.asarray(g, dtype=np.float64).reshape(ids.shape)
    lp, _, _ = log_softmax_rows(z)
    ids, ignored, bad, live = _slots(ids, V, ignore_index)
    K = ids.shape[1]
    with np.errstate(**_ERR):
        p = np.exp(lp)
    dz = np.zeros((n, V))
    for r in range(n):
        if not live[r].any() and not bad[r].any():
            continue  # every slot ignored: zero row
        if bad[r].any():
            dz[r] = np.nan
            continue
        G = 0.0
        for k in range(K):
            if live[r, k]:
                G += g[r, k]
                dz[r, ids[r, k]] += g[r, k]
        with np.errstate(**_ERR):
            dz[r] = dz[r] - G * p[r]
    return dz


def cond_logprobs_topk_fwd(z, ids, ignore_index=-100):
    """Conditioning scale per slot: |z_id - m| + |log S|."""
    z = np.asarray(z, dtype=np.float64)
    n, V = z.shape
    _, m, logS = log_softmax_rows(z)
    ids, ignored, bad, live = _slots(ids, V, ignore_index)
    c = np.repeat(np.abs(logS)[:, None], ids.shape[1], axis=1)
    with np.errstate(**_ERR):
        for r in range(n):
            for k in range(ids.shape[1]):
                if live[r, k]:
                    c[r, k] += abs(z[r, ids[r, k]] - m[r])
    return c


def cond_logprobs_topk_bwd(z, ids, g, ignore_index=-100):
    """sum_{k live, id = j} |g_k| + (sum_{k live} |g_k|) p_j (1 + |z_j - m| + |log S|)."""
    z = np.asarray(z, dtype=np.float64)
    n, V = z.shape
    g = np.abs(np.asarray(g, dtype=np.float64).reshape(ids.shape))
    lp, m, logS = log_softmax_rows(z)
    ids, ignored, bad, live = _slots(ids, V, ignore_index)
    with np.errstate(**_ERR):
        p = np.exp(lp)
        dzm = np.where(z > -np.inf, np.abs(z - m[:, None]), 0.0)
        c = np.zeros((n, V))
        for r in range(n):
            Ga = 0.0
            for k in range(ids.shape[1]):
                if live[r, k]:
                    Ga += g[r, k]
                    c[r, ids[r, k]] += g[r, k]
            c[r] += Ga * p[r] * (1.0 + dzm[r] + abs(logS[r]))
    return c
