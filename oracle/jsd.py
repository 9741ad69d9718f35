"""fp64 definition of the generalized Jensen-Shannon divergence (test infrastructure only).

Source: the JSD pull request whose text is pasted into DeepSpeed PR #8838
("Motivation", "Changes", "Scope and limitations"): a per-token divergence
``jsd(student_logits, teacher_logits, beta)`` for GKD-style distillation,
fp32 per token, gradients to both inputs, beta = 0 selecting forward KL and
beta = 1 reverse KL as explicit endpoint branches, interior 0 < beta < 1
computed, after a pass that gathers each input's statistics, from the KL of
each input to the mixture.

Reading taken (the page does not print the mixture): the generalized JSD of
GKD-style distillation that the page names, with S = student, T = teacher,

    M_j   = (1 - beta) p^S_j + beta p^T_j
    JSD   = beta KL(T || M) + (1 - beta) KL(S || M)          (0 < beta < 1)
    beta = 0:  KL(T || S)   (forward KL)
    beta = 1:  KL(S || T)   (reverse KL)

Endpoint branches use ``reductions.kl_fwd`` / ``kl_bwd`` with the arguments
in that order. Interior gradients, derived from the definition (the page
does not print them), with K_S = KL(S || M) and K_T = KL(T || M):

    dJSD/ds_k = (1 - beta) p^S_k ((log p^S_k - log M_k) - K_S)
    dJSD/dt_k = beta       p^T_k ((log p^T_k - log M_k) - K_T)

Entries equal to -inf have probability 0, add nothing and get gradient 0; so
does any term whose probability is exactly 0 in float64 (an underflow, as for
a row spanning -3e38..3e38), by the zero-weight rule of the "0 x inf" review
thread and its fix commit on PR #8838 (a weighted contribution whose weight is
zero is masked, never 0 x inf).
A row where either input is undefined (NaN, +inf, or no entry above -inf)
gives NaN and NaN gradients. Disjoint supports are finite in the interior
(the page tests "disjoint support").
"""

import numpy as np

from .reductions import kl_bwd, kl_fwd, log_softmax_rows, row_defined

__all__ = ["jsd_fwd", "jsd_bwd", "cond_jsd_fwd", "cond_jsd_bwd"]

_ERR = dict(invalid="ignore", over="ignore", divide="ignore", under="ignore")


def _interior(s, t, beta):
    """(p_s, p_t, ls, lt, lm, live_s, live_t, K_s, K_t, bad_rows) in float64."""
    s = np.asarray(s, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    ls, _, _ = log_softmax_rows(s)
    lt, _, _ = log_softmax_rows(t)
    live_s, live_t = s > -np.inf, t > -np.inf
    with np.errstate(**_ERR):
        ps, pt = np.exp(ls), np.exp(lt)
        M = (1.0 - beta) * ps + beta * pt
        lm = np.log(M)
        Ks = np.sum(np.where(ps > 0, ps * (ls - lm), 0.0), axis=1)
        Kt = np.sum(np.where(pt > 0, pt * (lt - lm), 0.0), axis=1)
    bad = ~row_defined(s) | ~row_defined(t)
    return ps, pt, ls, lt, lm, live_s, live_t, Ks, Kt, bad


def jsd_fwd(s, t, beta):
    """Per-row generalized JSD; returns (jsd [n], (K_S [n], K_T [n]) or None at the endpoints)."""
    beta = float(beta)
    if beta == 0.0:
        return kl_fwd(t, s)[0], None
    if beta == 1.0:
        return kl_fwd(s, t)[0], None
    _, _, _, _, _, _, _, Ks, Kt, bad = _interior(s, t, beta)
    with np.errstate(**_ERR):
        out = beta * Kt + (1.0 - beta) * Ks
    out[bad] = np.nan
    Ks = np.where(bad, np.nan, Ks)
    Kt = np.where(bad, np.nan, Kt)
    return out, (Ks, Kt)


def jsd_bwd(s, t, g, beta):
    """Gradients (ds, dt) of g * JSD_beta(S, T) per row."""
    beta = float(beta)
    n = np.asarray(s).shape[0]
    g = np.asarray(g, dtype=np.float64).reshape(n)
    if beta == 0.0:
        dt, ds = kl_bwd(t, s, g)
        return ds, dt
    if beta == 1.0:
        return kl_bwd(s, t, g)
    ps, pt, ls, lt, lm, live_s, live_t, Ks, Kt, bad = _interior(s, t, beta)
    with np.errstate(**_ERR):
        ds = np.where(ps > 0, g[:, None] * (1.0 - beta) * ps * ((ls - lm) - Ks[:, None]), 0.0)
        dt = np.where(pt > 0, g[:, None] * beta * pt * ((lt - lm) - Kt[:, None]), 0.0)
    ds[bad] = np.nan
    dt[bad] = np.nan
    return ds, dt


def cond_jsd_fwd(s, t, beta):
    """Conditioning scale per row: sum of the magnitudes the interior formula combines
    (|log p| + |log M| for each weighted term), or the KL scale at the endpoints."""
    from .reductions import cond_kl_fwd

    beta = float(beta)
    if beta == 0.0:
        return cond_kl_fwd(t, s)
    if beta == 1.0:
        return cond_kl_fwd(s, t)
    s = np.asarray(s, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    ps, pt, ls, lt, lm, live_s, live_t, _, _, _ = _interior(s, t, beta)
    _, ms, lss = log_softmax_rows(s)
    _, mt, lst = log_softmax_rows(t)
    with np.errstate(**_ERR):
        ws = np.where(ps > 0, ps * (np.abs(ls) + np.abs(lm) + np.abs(s - ms[:, None])), 0.0)
        wt = np.where(pt > 0, pt * (np.abs(lt) + np.abs(lm) + np.abs(t - mt[:, None])), 0.0)
        return np.sum(ws, axis=1) + np.sum(wt, axis=1) + np.abs(lss) + np.abs(lst)


def cond_jsd_bwd(s, t, g, beta):
    """Per-element scales (c_s, c_t): |g| w p (1 + |log p| + |log M| + |K| + centring terms)."""
    from .reductions import cond_kl_bwd

    beta = float(beta)
    if beta == 0.0:
        ct, cs = cond_kl_bwd(t, s, g)
        return cs, ct
    if beta == 1.0:
        return cond_kl_bwd(s, t, g)
    s = np.asarray(s, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    n = s.shape[0]
    g = np.abs(np.asarray(g, dtype=np.float64).reshape(n))
    ps, pt, ls, lt, lm, live_s, live_t, Ks, Kt, _ = _interior(s, t, beta)
    _, ms, lss = log_softmax_rows(s)
    _, mt, lst = log_softmax_rows(t)
    with np.errstate(**_ERR):
        base = 1.0 + np.abs(lm)
        cs = np.where(ps > 0, (1.0 - beta) * ps * (base + np.abs(s - ms[:, None]) + np.abs(lss)[:, None]
                                                   + np.abs(Ks)[:, None]), 0.0)
        ct = np.where(pt > 0, beta * pt * (base + np.abs(t - mt[:, None]) + np.abs(lst)[:, None]
                                           + np.abs(Kt)[:, None]), 0.0)
        # M mixes both inputs: each gradient also carries the other side's share of log M
        both = (ps > 0) & live_t
        cs = cs + np.where(both, (1.0 - beta) * ps * (np.abs(t - mt[:, None]) + np.abs(lst)[:, None]), 0.0)
        both = (pt > 0) & live_s
        ct = ct + np.where(both, beta * pt * (np.abs(s - ms[:, None]) + np.abs(lss)[:, None]), 0.0)
    cs = np.where(np.isnan(cs), 0.0, cs)
    ct = np.where(np.isnan(ct), 0.0, ct)
    return g[:, None] * cs, g[:, None] * ct
