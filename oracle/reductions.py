"""fp64 definitions of the per-row vocabulary reductions (test infrastructure only).

Source: DeepSpeed PR #8838 "Add Triton kernels for vocab-parallel logprobs,
entropy and KL". The ops are per-token log-probabilities, entropy and KL(A||B)
over one row of logits, returning one fp32 value per token (JSD squash-commit
text, "Changes"); gradients are returned per logit (second commit message).

Everything here is the plain definition, evaluated in float64 with two passes
over each row (max, then sums). Inputs are upcast exactly (bf16 and fp32
values are exactly representable in float64). Where the pages leave a value
open, the reading taken is stated in the function's docstring:

* a row is *defined* when it has no NaN, no +inf and at least one entry
  above -inf; an undefined row yields NaN outputs and NaN gradients (the
  pages list all -inf rows as a test case without giving the value; NaN is
  what a dense log_softmax produces there);
* an entry equal to -inf is masked: it has probability 0, it is left out of
  every sum, and its gradient is 0 (the zero-weight rule of the "0 x inf"
  review thread and its fix commit);
* ``ignore_index`` gives output 0 and a zero gradient row; a target outside
  [0, V) that is not ignored gives NaN (no status can be raised without a
  host synchronisation);
* KL(A||B) is +inf when B masks (-inf) a column that A supports (A > -inf):
  the support-mismatch flag is decided on the logits, not on the computed
  probabilities (second commit message; review comment). For such a row the
  gradient with respect to A is NaN in every column (the derivative of an
  infinite loss is undefined) and the gradient with respect to B is the
  term-wise g (p_B - p_A).
"""

import numpy as np

__all__ = [
    "row_defined",
    "log_softmax_rows",
    "logprobs_fwd",
    "logprobs_bwd",
    "entropy_fwd",
    "entropy_bwd",
    "kl_fwd",
    "kl_bwd",
    "single_read_identities",
    "cond_logprobs_fwd",
    "cond_entropy_fwd",
    "cond_kl_fwd",
    "cond_logprobs_bwd",
    "cond_entropy_bwd",
    "cond_kl_bwd",
]

_ERR = dict(invalid="ignore", over="ignore", divide="ignore", under="ignore")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def row_defined(z):
    """True for rows with no NaN, no +inf and at least one entry above -inf."""
    z = _f64(z)
    return (~np.isnan(z).any(axis=1)) & (~np.isposinf(z).any(axis=1)) & (z > -np.inf).any(axis=1)


def log_softmax_rows(z):
    """Per-row log-softmax by its definition.

    m = max_j z_j, S = sum_j exp(z_j - m), log p_j = (z_j - m) - log S.
    Returns (logp [n, V], m [n], logS [n]); undefined rows are NaN throughout.
    """
    z = _f64(z)
    ok = row_defined(z)
    with np.errstate(**_ERR):
        m = np.max(z, axis=1)
        d = z - m[:, None]
        S = np.sum(np.exp(d), axis=1)
        logS = np.log(S)
        logp = d - logS[:, None]
    logp[~ok] = np.nan
    m = np.where(ok, m, np.nan)
    logS = np.where(ok, logS, np.nan)
    return logp, m, logS


def _target_state(t, V, ignore_index):
    t = np.asarray(t, dtype=np.int64)
    ignored = t == ignore_index
    in_range = (t >= 0) & (t < V)
    return t, ignored, in_range


def logprobs_fwd(z, t, ignore_index=-100):
    """Per-token log-probability log p_t of the target column.

    Returns (logp [n], m [n], logS [n]). Ignored rows give 0; a target outside
    [0, V) that is not ignored, or an undefined row, gives NaN.
    """
    z = _f64(z)
    n, V = z.shape
    lp, m, logS = log_softmax_rows(z)
    t, ignored, in_range = _target_state(t, V, ignore_index)
    out = np.full(n, np.nan)
    sel = in_range & ~ignored
    rows = np.nonzero(sel)[0]
    out[rows] = lp[rows, t[rows]]
    out[ignored] = 0.0
    return out, m, logS


def logprobs_bwd(z, t, g, ignore_index=-100):
    """d logp_t / d z_j times g: g (1[j = t] - p_j).

    This is the gradient of RL-Kernel PR #208 (review nitpick on the chunked
    backward: the negated probabilities, one added at the target column, all
    scaled by the upstream gradient).
    Ignored rows are all zero; out-of-range targets and undefined rows NaN.
    """
    z = _f64(z)
    n, V = z.shape
    g = _f64(g).reshape(n)
    lp, _, _ = log_softmax_rows(z)
    t, ignored, in_range = _target_state(t, V, ignore_index)
    with np.errstate(**_ERR):
        p = np.exp(lp)
        dz = -p
        rows = np.nonzero(in_range & ~ignored)[0]
        dz[rows, t[rows]] += 1.0
        dz = dz * g[:, None]
    dz[~in_range & ~ignored] = np.nan
    dz[ignored] = 0.0
    return dz


def entropy_fwd(z):
    """H = -sum_{j: z_j > -inf} p_j log p_j. Returns (H [n], m [n], logS [n])."""
    z = _f64(z)
    lp, m, logS = log_softmax_rows(z)
    live = z > -np.inf
    with np.errstate(**_ERR):
        p = np.exp(lp)
        terms = np.where(live, p * lp, 0.0)
        H = -np.sum(terms, axis=1)
    H[~row_defined(z)] = np.nan
    return H, m, logS


def entropy_bwd(z, g):
    """dH/dz_j times g: -g p_j (log p_j + H); exactly 0 where z_j = -inf.

    Derived from the definition (the pages do not print it): with
    H = -sum p log p and dp_k/dz_j = p_k (1[k=j] - p_j),
    dH/dz_j = -p_j (log p_j + 1) + p_j sum_k p_k (log p_k + 1) = -p_j (log p_j + H).
    """
    z = _f64(z)
    n, V = z.shape
    g = _f64(g).reshape(n)
    lp, _, _ = log_softmax_rows(z)
    H, _, _ = entropy_fwd(z)
    live = z > -np.inf
    with np.errstate(**_ERR):
        p = np.exp(lp)
        dz = np.where(live, -g[:, None] * p * (lp + H[:, None]), 0.0)
    dz[~row_defined(z)] = np.nan
    return dz


def _kl_row_state(a, b):
    """(value_nan rows, F rows) for KL(A||B).

    NaN when A is undefined, or B holds a NaN or +inf. F (support mismatch):
    some column has a_j > -inf and b_j = -inf.
    """
    nan_rows = ~row_defined(a) | np.isnan(b).any(axis=1) | np.isposinf(b).any(axis=1)
    F = ((a > -np.inf) & (b == -np.inf)).any(axis=1)
    return nan_rows, F & ~nan_rows


def kl_fwd(a, b):
    """KL(A||B) = sum_{j: a_j > -inf} p^A_j (log p^A_j - log p^B_j); +inf when F.

    Returns (kl [n], (m_a, logS_a, m_b, logS_b)).
    """
    a = _f64(a)
    b = _f64(b)
    lpa, ma, lsa = log_softmax_rows(a)
    lpb, mb, lsb = log_softmax_rows(b)
    nan_rows, F = _kl_row_state(a, b)
    live = a > -np.inf
    with np.errstate(**_ERR):
        pa = np.exp(lpa)
        terms = np.where(live, pa * (lpa - lpb), 0.0)
        kl = np.sum(terms, axis=1)
    kl[F] = np.inf
    kl[nan_rows] = np.nan
    return kl, (ma, lsa, mb, lsb)


def kl_bwd(a, b, g):
    """Gradients of g * KL(A||B).

    dKL/da_j = p^A_j (log p^A_j - log p^B_j - KL), exactly 0 where a_j = -inf;
    dKL/db_j = p^B_j - p^A_j. Derived from the definition (the pages do not
    print them). Rows with F: grad_a is NaN in every column, grad_b stays
    g (p_B - p_A). Rows whose KL is NaN: both gradients NaN.
    Returns (da, db).
    """
    a = _f64(a)
    b = _f64(b)
    n, V = a.shape
    g = _f64(g).reshape(n)
    lpa, _, _ = log_softmax_rows(a)
    lpb, _, _ = log_softmax_rows(b)
    kl, _ = kl_fwd(a, b)
    nan_rows, F = _kl_row_state(a, b)
    live = a > -np.inf
    with np.errstate(**_ERR):
        pa = np.exp(lpa)
        pb = np.exp(lpb)
        da = np.where(live, g[:, None] * pa * (lpa - lpb - kl[:, None]), 0.0)
        db = g[:, None] * (pb - pa)
    da[F] = np.nan
    da[nan_rows] = np.nan
    db[nan_rows] = np.nan
    return da, db


def single_read_identities(z, b=None):
    """The single-read statistics of the pages, evaluated in float64.

    With m the row max, S = sum e^(z-m), W_H = sum e^(z-m)(z-m):
    H = log S - W_H/S. With W_K = sum e^(a-m_a)((a-m_a)-(b-m_b)):
    KL = W_K/S_A - log S_A + log S_B (PR #8838, second commit message).
    Only used to cross-check the definitions above; masked (-inf) columns are
    left out of W (zero-weight rule). Returns H, or (H_a, KL) when b is given.
    """
    z = _f64(z)
    with np.errstate(**_ERR):
        m = np.max(z, axis=1, keepdims=True)
        d = z - m
        e = np.exp(d)
        S = e.sum(axis=1)
        W = np.where(z > -np.inf, e * d, 0.0).sum(axis=1)
        H = np.log(S) - W / S
        if b is None:
            return H
        b = _f64(b)
        mb = np.max(b, axis=1, keepdims=True)
        db = b - mb
        SB = np.exp(db).sum(axis=1)
        WK = np.where(z > -np.inf, e * (d - db), 0.0).sum(axis=1)
        KL = WK / S - np.log(S) + np.log(SB)
    return H, KL


# ---------------------------------------------------------------------------
# Conditioning scales: for each output element, the sum of magnitudes of the
# terms its formula combines. They scale the rounding allowance of the parity
# rule (an exact result that is a near-cancelling difference cannot be held to
# a purely relative bound).
# ---------------------------------------------------------------------------


def _cent(z):
    """(p, |z - m|, |log S|) per element / row, zero-weight entries masked."""
    z = _f64(z)
    lp, m, logS = log_softmax_rows(z)
    with np.errstate(**_ERR):
        p = np.exp(lp)
        dz = np.where(z > -np.inf, np.abs(z - m[:, None]), 0.0)
    return p, dz, np.abs(logS)


def cond_logprobs_fwd(z, t, ignore_index=-100):
    """|z_t - m| + |log S|."""
    z = _f64(z)
    n, V = z.shape
    _, dz, als = _cent(z)
    t, ignored, in_range = _target_state(t, V, ignore_index)
    c = np.array(als)
    rows = np.nonzero(in_range & ~ignored)[0]
    c[rows] += dz[rows, t[rows]]
    return c


def cond_entropy_fwd(z):
    """|log S| + sum_j p_j |z_j - m|."""
    p, dz, als = _cent(z)
    with np.errstate(**_ERR):
        return als + np.sum(np.where(np.isfinite(dz), p * dz, 0.0), axis=1)


def cond_kl_fwd(a, b):
    """sum_j p^A_j (|a_j - m_a| + |b_j - m_b|) + |log S_A| + |log S_B|."""
    pa, da, lsa = _cent(a)
    _, db, lsb = _cent(b)
    with np.errstate(**_ERR):
        w = np.where(np.isfinite(da) & np.isfinite(db), pa * (da + db), 0.0)
    return np.sum(w, axis=1) + lsa + lsb


def cond_logprobs_bwd(z, t, g, ignore_index=-100):
    """|g| (1[j=t] + p_j (1 + |z_j - m| + |log S|))."""
    z = _f64(z)
    n, V = z.shape
    g = np.abs(_f64(g).reshape(n))
    p, dz, als = _cent(z)
    t, ignored, in_range = _target_state(t, V, ignore_index)
    with np.errstate(**_ERR):
        c = p * (1.0 + dz + als[:, None])
        rows = np.nonzero(in_range & ~ignored)[0]
        c[rows, t[rows]] += 1.0
        return g[:, None] * c


def cond_entropy_bwd(z, g):
    """|g| p_j (1 + |z_j - m| + |log S| + |H|)."""
    z = _f64(z)
    n, V = z.shape
    g = np.abs(_f64(g).reshape(n))
    p, dz, als = _cent(z)
    H, _, _ = entropy_fwd(z)
    with np.errstate(**_ERR):
        return g[:, None] * p * (1.0 + dz + als[:, None] + np.abs(H)[:, None])


def cond_kl_bwd(a, b, g):
    """grad_a: |g| p^A (1 + |a-m_a| + |b-m_b| + |log S_A| + |log S_B| + |KL|);
    grad_b: |g| (p^A (1 + |a-m_a| + |log S_A|) + p^B (1 + |b-m_b| + |log S_B|))."""
    a = _f64(a)
    n, V = a.shape
    g = np.abs(_f64(g).reshape(n))
    pa, da, lsa = _cent(a)
    pb, db, lsb = _cent(b)
    kl, _ = kl_fwd(a, b)
    with np.errstate(**_ERR):
        ca = g[:, None] * pa * (1.0 + da + db + lsa[:, None] + lsb[:, None] + np.abs(kl)[:, None])
        cb = g[:, None] * (pa * (1.0 + da + lsa[:, None]) + pb * (1.0 + db + lsb[:, None]))
    return ca, cb
