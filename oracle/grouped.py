"""Count-weighted forms of the per-row reductions for rows made of repeated values.

Test infrastructure only: nothing outside tests/ (and the smoke check / the CPU
baseline) may import this package.

A row of V logits that holds only k distinct (a_i, b_i) pairs, pair i repeated
cnt_i times, has every sum in the definitions of oracle.reductions equal to a
count-weighted sum over the k pairs, and every gradient entry equal to the value
of its pair. These forms let a test check rows far wider than the host could
hold as float64 arrays -- up to the widest row the library accepts -- against
the same definitions: per-token log-probability, entropy and KL(A||B) of
DeepSpeed PR #8838 "Add Triton kernels for vocab-parallel logprobs, entropy and
KL" (ops listed in the JSD squash-commit text; gradients per logit, second
commit message), the logprobs gradient printed in the review nitpick of
RL-Kernel PR #208, and the multi-id (top-k) form whose duplicate and ignored
ids that PR's test list names, and the generalized JSD of the JSD pull request
pasted into PR #8838 (the GKD-style mixture read in oracle.jsd). The readings
are those of oracle.reductions, oracle.topk and oracle.jsd: -inf entries are masked (probability 0, left out of every sum,
zero gradient); a row with a NaN or +inf entry or no entry above -inf is
undefined (NaN); KL(A||B) is +inf when B masks a column A supports, with a NaN
gradient for A.

A target or a top-k id names one column; its pair must be a group of its own
(cnt 1), since the one-hot term tells that column apart from the others of the
same value. Every function takes one row: z (or a, b) [k] values and cnt [k]
positive integer counts, and returns per-group values for the gradients.

Pinned in tests/test_oracle_grouped.py against oracle.reductions, oracle.topk
and oracle.jsd on the same rows expanded to dense form.
"""

import numpy as np

__all__ = [
    "log_softmax",
    "logprobs_fwd",
    "logprobs_bwd",
    "entropy_fwd",
    "entropy_bwd",
    "kl_fwd",
    "kl_bwd",
    "logprobs_topk_fwd",
    "logprobs_topk_bwd",
    "cond_logprobs_fwd",
    "cond_logprobs_bwd",
    "cond_entropy_fwd",
    "cond_entropy_bwd",
    "cond_kl_fwd",
    "cond_kl_bwd",
    "cond_logprobs_topk_fwd",
    "cond_logprobs_topk_bwd",
    "jsd_fwd",
    "jsd_bwd",
    "cond_jsd_fwd",
    "cond_jsd_bwd",
]

_ERR = dict(invalid="ignore", over="ignore", divide="ignore", under="ignore")


def _row(z, cnt):
    z = np.asarray(z, dtype=np.float64).reshape(-1)
    cnt = np.asarray(cnt, dtype=np.float64).reshape(-1)
    if z.shape != cnt.shape or not (cnt >= 1).all() or not (cnt == np.floor(cnt)).all():
        raise ValueError("one value and one positive integer count per group")
    return z, cnt


def _defined(z):
    return not np.isnan(z).any() and not np.isposinf(z).any() and (z > -np.inf).any()


def _single(cnt, i):
    if cnt[i] != 1:
        raise ValueError("a target column must be a group of its own (count 1)")


def log_softmax(z, cnt):
    """(log p per group, m, log S): m = max z, S = sum_i cnt_i exp(z_i - m); NaN when undefined."""
    z, cnt = _row(z, cnt)
    if not _defined(z):
        return np.full(z.shape, np.nan), np.nan, np.nan
    m = np.max(z)
    with np.errstate(**_ERR):
        d = z - m
        logS = np.log(np.sum(cnt * np.exp(d)))
        return d - logS, m, logS


def logprobs_fwd(z, cnt, t):
    """(log p of the target's group t, m, log S)."""
    z, cnt = _row(z, cnt)
    _single(cnt, t)
    lp, m, logS = log_softmax(z, cnt)
    return lp[t], m, logS


def logprobs_bwd(z, cnt, t, g):
    """Per group: g (1[group = t] - p)."""
    z, cnt = _row(z, cnt)
    _single(cnt, t)
    lp, _, _ = log_softmax(z, cnt)
    with np.errstate(**_ERR):
        dz = -np.exp(lp)
        dz[t] += 1.0
        return dz * float(g)


def entropy_fwd(z, cnt):
    """(H = -sum over live groups of cnt p log p, m, log S)."""
    z, cnt = _row(z, cnt)
    lp, m, logS = log_softmax(z, cnt)
    if np.isnan(m):
        return np.nan, m, logS
    live = z > -np.inf
    with np.errstate(**_ERR):
        H = -np.sum(np.where(live, cnt * np.exp(lp) * lp, 0.0))
    return H, m, logS


def entropy_bwd(z, cnt, g):
    """Per group: -g p (log p + H); 0 for masked groups."""
    z, cnt = _row(z, cnt)
    lp, _, _ = log_softmax(z, cnt)
    H, _, _ = entropy_fwd(z, cnt)
    if np.isnan(H):
        return np.full(z.shape, np.nan)
    with np.errstate(**_ERR):
        return np.where(z > -np.inf, -float(g) * np.exp(lp) * (lp + H), 0.0)


def _kl_state(a, b):
    nan_row = not _defined(a) or np.isnan(b).any() or np.isposinf(b).any()
    F = bool(((a > -np.inf) & (b == -np.inf)).any())
    return nan_row, F and not nan_row


def kl_fwd(a, b, cnt):
    """(KL(A||B) = sum over groups with a > -inf of cnt p_A (log p_A - log p_B); +inf on a
    support mismatch, (m_a, log S_A, m_b, log S_B))."""
    a, cnt = _row(a, cnt)
    b, _ = _row(b, cnt)
    lpa, ma, lsa = log_softmax(a, cnt)
    lpb, mb, lsb = log_softmax(b, cnt)
    nan_row, F = _kl_state(a, b)
    if nan_row:
        return np.nan, (ma, lsa, mb, lsb)
    if F:
        return np.inf, (ma, lsa, mb, lsb)
    with np.errstate(**_ERR):
        kl = np.sum(np.where(a > -np.inf, cnt * np.exp(lpa) * (lpa - lpb), 0.0))
    return kl, (ma, lsa, mb, lsb)


def kl_bwd(a, b, cnt, g):
    """Per group: (g p_A (log p_A - log p_B - KL), 0 where a = -inf; g (p_B - p_A)).
    A support mismatch makes the first NaN in every group; an undefined row both."""
    a, cnt = _row(a, cnt)
    b, _ = _row(b, cnt)
    lpa, _, _ = log_softmax(a, cnt)
    lpb, _, _ = log_softmax(b, cnt)
    kl, _ = kl_fwd(a, b, cnt)
    nan_row, F = _kl_state(a, b)
    g = float(g)
    with np.errstate(**_ERR):
        pa, pb = np.exp(lpa), np.exp(lpb)
        da = np.where(a > -np.inf, g * pa * (lpa - lpb - kl), 0.0)
        db = g * (pb - pa)
    if F or nan_row:
        da = np.full(a.shape, np.nan)
    if nan_row:
        db = np.full(a.shape, np.nan)
    return da, db


def logprobs_topk_fwd(z, cnt, slots):
    """(log p of each slot's group, m, log S); slots [K] group indexes, each a group of its own."""
    z, cnt = _row(z, cnt)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    for s in slots:
        _single(cnt, s)
    lp, m, logS = log_softmax(z, cnt)
    return lp[slots], m, logS


def logprobs_topk_bwd(z, cnt, slots, gk):
    """Per group: h - G p, with h the sum of the slot gradients gk naming the group (duplicates
    add) and G the sum of all of them."""
    z, cnt = _row(z, cnt)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    gk = np.asarray(gk, dtype=np.float64).reshape(-1)
    for s in slots:
        _single(cnt, s)
    lp, _, _ = log_softmax(z, cnt)
    h = np.zeros(z.shape)
    np.add.at(h, slots, gk)
    with np.errstate(**_ERR):
        return h - np.sum(gk) * np.exp(lp)


# ---- conditioning scales: the count-weighted forms of those in oracle.reductions / oracle.topk


def _cent(z, cnt):
    lp, m, logS = log_softmax(z, cnt)
    with np.errstate(**_ERR):
        p = np.exp(lp)
        dz = np.where(z > -np.inf, np.abs(z - m), 0.0)
    return p, dz, abs(logS)


def cond_logprobs_fwd(z, cnt, t):
    """|z_t - m| + |log S|."""
    z, cnt = _row(z, cnt)
    _, dz, als = _cent(z, cnt)
    return als + dz[t]


def cond_logprobs_bwd(z, cnt, t, g):
    """Per group: |g| (1[group = t] + p (1 + |z - m| + |log S|))."""
    z, cnt = _row(z, cnt)
    p, dz, als = _cent(z, cnt)
    with np.errstate(**_ERR):
        c = p * (1.0 + dz + als)
    c[t] += 1.0
    return abs(float(g)) * c


def cond_entropy_fwd(z, cnt):
    """|log S| + sum_i cnt_i p_i |z_i - m|."""
    z, cnt = _row(z, cnt)
    p, dz, als = _cent(z, cnt)
    with np.errstate(**_ERR):
        return als + np.sum(np.where(np.isfinite(dz), cnt * p * dz, 0.0))


def cond_entropy_bwd(z, cnt, g):
    """Per group: |g| p (1 + |z - m| + |log S| + |H|)."""
    z, cnt = _row(z, cnt)
    p, dz, als = _cent(z, cnt)
    H, _, _ = entropy_fwd(z, cnt)
    with np.errstate(**_ERR):
        return abs(float(g)) * p * (1.0 + dz + als + abs(H))


def cond_kl_fwd(a, b, cnt):
    """sum_i cnt_i p_A,i (|a_i - m_a| + |b_i - m_b|) + |log S_A| + |log S_B|."""
    a, cnt = _row(a, cnt)
    b, _ = _row(b, cnt)
    pa, da, lsa = _cent(a, cnt)
    _, db, lsb = _cent(b, cnt)
    with np.errstate(**_ERR):
        w = np.where(np.isfinite(da) & np.isfinite(db), cnt * pa * (da + db), 0.0)
    return np.sum(w) + lsa + lsb


def cond_kl_bwd(a, b, cnt, g):
    """Per group: grad_a |g| p_A (1 + |a - m_a| + |b - m_b| + |log S_A| + |log S_B| + |KL|);
    grad_b |g| (p_A (1 + |a - m_a| + |log S_A|) + p_B (1 + |b - m_b| + |log S_B|))."""
    a, cnt = _row(a, cnt)
    b, _ = _row(b, cnt)
    pa, da, lsa = _cent(a, cnt)
    pb, db, lsb = _cent(b, cnt)
    kl, _ = kl_fwd(a, b, cnt)
    g = abs(float(g))
    with np.errstate(**_ERR):
        ca = g * pa * (1.0 + da + db + lsa + lsb + abs(kl))
        cb = g * (pa * (1.0 + da + lsa) + pb * (1.0 + db + lsb))
    return ca, cb


def cond_logprobs_topk_fwd(z, cnt, slots):
    """Per slot: |z_id - m| + |log S|."""
    z, cnt = _row(z, cnt)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    _, dz, als = _cent(z, cnt)
    return als + dz[slots]


def cond_logprobs_topk_bwd(z, cnt, slots, gk):
    """Per group: sum of |g_k| over the slots naming it + (sum_k |g_k|) p (1 + |z - m| + |log S|)."""
    z, cnt = _row(z, cnt)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    ga = np.abs(np.asarray(gk, dtype=np.float64).reshape(-1))
    p, dz, als = _cent(z, cnt)
    c = np.zeros(z.shape)
    np.add.at(c, slots, ga)
    with np.errstate(**_ERR):
        return c + np.sum(ga) * p * (1.0 + dz + als)


# ---- generalized JSD (student s, teacher t): M = (1 - beta) p_S + beta p_T,
# JSD = beta KL(T||M) + (1 - beta) KL(S||M) inside (0, 1); KL(T||S) at beta = 0, KL(S||T) at 1


def _jsd_interior(s, t, cnt, beta):
    ls, ms, lss = log_softmax(s, cnt)
    lt, mt, lst = log_softmax(t, cnt)
    with np.errstate(**_ERR):
        ps, pt = np.exp(ls), np.exp(lt)
        lm = np.log((1.0 - beta) * ps + beta * pt)
        Ks = np.sum(np.where(ps > 0, cnt * ps * (ls - lm), 0.0))
        Kt = np.sum(np.where(pt > 0, cnt * pt * (lt - lm), 0.0))
    bad = not _defined(s) or not _defined(t)
    return ps, pt, ls, lt, lm, Ks, Kt, bad, (ms, lss, mt, lst)


def jsd_fwd(s, t, cnt, beta):
    """(JSD, (K_S, K_T) inside (0, 1), None at the endpoints)."""
    s, cnt = _row(s, cnt)
    t, _ = _row(t, cnt)
    beta = float(beta)
    if beta == 0.0:
        return kl_fwd(t, s, cnt)[0], None
    if beta == 1.0:
        return kl_fwd(s, t, cnt)[0], None
    _, _, _, _, _, Ks, Kt, bad, _ = _jsd_interior(s, t, cnt, beta)
    if bad:
        return np.nan, (np.nan, np.nan)
    return beta * Kt + (1.0 - beta) * Ks, (Ks, Kt)


def jsd_bwd(s, t, cnt, g, beta):
    """Per group: (g (1 - beta) p_S ((log p_S - log M) - K_S), g beta p_T ((log p_T - log M) - K_T)),
    0 where the probability is 0; the KL gradients at the endpoints."""
    s, cnt = _row(s, cnt)
    t, _ = _row(t, cnt)
    beta, g = float(beta), float(g)
    if beta == 0.0:
        dt, ds = kl_bwd(t, s, cnt, g)
        return ds, dt
    if beta == 1.0:
        return kl_bwd(s, t, cnt, g)
    ps, pt, ls, lt, lm, Ks, Kt, bad, _ = _jsd_interior(s, t, cnt, beta)
    if bad:
        return np.full(s.shape, np.nan), np.full(s.shape, np.nan)
    with np.errstate(**_ERR):
        ds = np.where(ps > 0, g * (1.0 - beta) * ps * ((ls - lm) - Ks), 0.0)
        dt = np.where(pt > 0, g * beta * pt * ((lt - lm) - Kt), 0.0)
    return ds, dt


def cond_jsd_fwd(s, t, cnt, beta):
    """Count-weighted form of oracle.jsd.cond_jsd_fwd."""
    s, cnt = _row(s, cnt)
    t, _ = _row(t, cnt)
    beta = float(beta)
    if beta == 0.0:
        return cond_kl_fwd(t, s, cnt)
    if beta == 1.0:
        return cond_kl_fwd(s, t, cnt)
    ps, pt, ls, lt, lm, _, _, _, (ms, lss, mt, lst) = _jsd_interior(s, t, cnt, beta)
    with np.errstate(**_ERR):
        ws = np.where(ps > 0, cnt * ps * (np.abs(ls) + np.abs(lm) + np.abs(s - ms)), 0.0)
        wt = np.where(pt > 0, cnt * pt * (np.abs(lt) + np.abs(lm) + np.abs(t - mt)), 0.0)
        return np.sum(ws) + np.sum(wt) + abs(lss) + abs(lst)


def cond_jsd_bwd(s, t, cnt, g, beta):
    """Count-weighted form of oracle.jsd.cond_jsd_bwd: per group (c_s, c_t)."""
    s, cnt = _row(s, cnt)
    t, _ = _row(t, cnt)
    beta = float(beta)
    if beta == 0.0:
        ct, cs = cond_kl_bwd(t, s, cnt, g)
        return cs, ct
    if beta == 1.0:
        return cond_kl_bwd(s, t, cnt, g)
    g = abs(float(g))
    ps, pt, ls, lt, lm, Ks, Kt, _, (ms, lss, mt, lst) = _jsd_interior(s, t, cnt, beta)
    live_s, live_t = s > -np.inf, t > -np.inf
    with np.errstate(**_ERR):
        base = 1.0 + np.abs(lm)
        cs = np.where(ps > 0, (1.0 - beta) * ps * (base + np.abs(s - ms) + abs(lss) + abs(Ks)), 0.0)
        ct = np.where(pt > 0, beta * pt * (base + np.abs(t - mt) + abs(lst) + abs(Kt)), 0.0)
        # the other side's share of log M
        cs = cs + np.where((ps > 0) & live_t, (1.0 - beta) * ps * (np.abs(t - mt) + abs(lst)), 0.0)
        ct = ct + np.where((pt > 0) & live_s, beta * pt * (np.abs(s - ms) + abs(lss)), 0.0)
    cs = np.where(np.isnan(cs), 0.0, cs)
    ct = np.where(np.isnan(ct), 0.0, ct)
    return g * cs, g * ct
