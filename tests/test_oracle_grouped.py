"""Pins of oracle.grouped (count-weighted forms for rows of repeated values) against the dense
definitions of oracle.reductions, oracle.topk and oracle.jsd (CPU only).

Every grouped row is expanded to its dense form (each value repeated its count times) and every
output, saved statistic, per-column gradient and conditioning scale of the grouped forms must
equal the dense one to 1e-12 relative. Counts above 1 in every row, masked (-inf) groups, an
offset row (+1e4), a row with one dominant entry, a support mismatch (+inf KL, NaN gradient
for A), an undefined row and duplicate top-k slots are covered, so a dropped count weight, a
wrong sign or a term left out of a sum fails here.
"""

import numpy as np
import pytest

from oracle import grouped as Gr, jsd as J, reductions as R, topk as TK

NINF = -np.inf


def _close(x, y, label, scale=None):
    """|x - y| <= 1e-12 max(|y|, scale): both sides sum the same terms in another order, so they
    differ by rounding of the terms' size, which the conditioning scale bounds where the result
    is a near-cancelling difference."""
    x, y = np.asarray(x, dtype=np.float64), np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (label, x.shape, y.shape)
    nan = np.isnan(x) | np.isnan(y)
    assert (np.isnan(x) == np.isnan(y)).all(), (label, x, y)
    inf = np.isinf(x) | np.isinf(y)
    assert (x[inf] == y[inf]).all(), (label, x[inf], y[inf])
    ok = ~nan & ~inf
    ref = np.abs(y) if scale is None else np.maximum(np.abs(y), np.nan_to_num(np.asarray(scale, dtype=np.float64)))
    err = np.abs(x[ok] - y[ok])
    assert (err <= 1e-12 * ref[ok] + 1e-300).all(), (label, np.max(err))


def _rows():
    """(a, b, cnt, t, slots, label): t and slots index count-1 groups."""
    rng = np.random.default_rng(7)
    out = []
    for i in range(6):
        k = 9
        a = rng.normal(0, 3, k)
        b = a + rng.normal(0, 0.7, k)
        cnt = rng.integers(2, 40, k)
        cnt[[0, 3, 5]] = 1  # count-1 groups for the target and the slots
        if i % 2:
            a[7] = b[7] = NINF  # a masked group in both
        if i == 2:
            a += 1e4
            b += 1e4
        if i == 4:
            a[0] = 30.0  # one dominant entry
        out.append((a, b, cnt, 3, np.array([0, 5, 3, 5]), "random %d" % i))
    a = np.array([1.0, 0.5, -2.0, 0.0, 3.0])
    b = np.array([0.0, NINF, 1.0, 2.0, 1.0])  # B masks a column A supports
    out.append((a, b, np.array([1, 4, 7, 1, 2]), 0, np.array([0, 3]), "support mismatch"))
    a = np.array([NINF, NINF, NINF])
    out.append((a, np.zeros(3), np.array([1, 5, 2]), 0, np.array([0]), "all masked"))
    return out


def _dense(a, b, cnt, t, slots):
    col = np.concatenate([[0], np.cumsum(cnt)[:-1]])  # first column of each group
    return np.repeat(a, cnt)[None], np.repeat(b, cnt)[None], col[t], col[slots]


@pytest.mark.parametrize("case", range(len(_rows())))
def test_grouped_matches_dense(case):
    a, b, cnt, t, slots, label = _rows()[case]
    da, db, tc, sc = _dense(a, b, cnt, t, slots)
    g, gk = 0.75, np.array([0.5, -1.25, 2.0, 0.25])[: len(slots)]
    rep = lambda v: np.repeat(np.asarray(v, dtype=np.float64), cnt)

    lp, m, ls = Gr.logprobs_fwd(a, cnt, t)
    rlp, rm, rls = R.logprobs_fwd(da, [tc])
    _close([lp, m, ls], [rlp[0], rm[0], rls[0]], label + " logprobs fwd")
    _close(rep(Gr.logprobs_bwd(a, cnt, t, g)), R.logprobs_bwd(da, [tc], [g])[0], label + " logprobs bwd",
           R.cond_logprobs_bwd(da, [tc], [g])[0])
    H, _, _ = Gr.entropy_fwd(a, cnt)
    _close(H, R.entropy_fwd(da)[0][0], label + " entropy fwd", R.cond_entropy_fwd(da)[0])
    _close(rep(Gr.entropy_bwd(a, cnt, g)), R.entropy_bwd(da, [g])[0], label + " entropy bwd",
           R.cond_entropy_bwd(da, [g])[0])
    for x, y, xd, yd, d in ((a, b, da, db, "A||B"), (b, a, db, da, "B||A")):
        kl, st = Gr.kl_fwd(x, y, cnt)
        rkl, rst = R.kl_fwd(xd, yd)
        _close([kl] + list(st), [rkl[0]] + [s[0] for s in rst], label + " kl fwd " + d,
               [R.cond_kl_fwd(xd, yd)[0], 0, 0, 0, 0])
        gx, gy = Gr.kl_bwd(x, y, cnt, g)
        rx, ry = R.kl_bwd(xd, yd, [g])
        scx, scy = R.cond_kl_bwd(xd, yd, [g])
        _close(rep(gx), rx[0], label + " kl bwd a " + d, scx[0])
        _close(rep(gy), ry[0], label + " kl bwd b " + d, scy[0])
        _close(Gr.cond_kl_fwd(x, y, cnt), R.cond_kl_fwd(xd, yd)[0], label + " cond kl fwd " + d)
        cx, cy = Gr.cond_kl_bwd(x, y, cnt, g)
        rcx, rcy = R.cond_kl_bwd(xd, yd, [g])
        _close(rep(cx), rcx[0], label + " cond kl bwd a " + d)
        _close(rep(cy), rcy[0], label + " cond kl bwd b " + d)
    out, _, _ = Gr.logprobs_topk_fwd(a, cnt, slots)
    _close(out, TK.logprobs_topk_fwd(da, sc[None])[0][0], label + " topk fwd")
    _close(rep(Gr.logprobs_topk_bwd(a, cnt, slots, gk)), TK.logprobs_topk_bwd(da, sc[None], gk[None])[0],
           label + " topk bwd", TK.cond_logprobs_topk_bwd(da, sc[None], gk[None])[0])
    if np.isfinite(m):  # the scales of undefined rows are NaN on both sides, not compared
        _close(Gr.cond_logprobs_fwd(a, cnt, t), R.cond_logprobs_fwd(da, [tc])[0], label + " cond logprobs fwd")
        _close(rep(Gr.cond_logprobs_bwd(a, cnt, t, g)), R.cond_logprobs_bwd(da, [tc], [g])[0],
               label + " cond logprobs bwd")
        _close(Gr.cond_entropy_fwd(a, cnt), R.cond_entropy_fwd(da)[0], label + " cond entropy fwd")
        _close(rep(Gr.cond_entropy_bwd(a, cnt, g)), R.cond_entropy_bwd(da, [g])[0], label + " cond entropy bwd")
        _close(Gr.cond_logprobs_topk_fwd(a, cnt, slots), TK.cond_logprobs_topk_fwd(da, sc[None])[0],
               label + " cond topk fwd")
        _close(rep(Gr.cond_logprobs_topk_bwd(a, cnt, slots, gk)), TK.cond_logprobs_topk_bwd(da, sc[None], gk[None])[0],
               label + " cond topk bwd")


@pytest.mark.parametrize("beta", [0.0, 0.3, 0.5, 1.0])
@pytest.mark.parametrize("case", range(len(_rows())))
def test_grouped_jsd_matches_dense(case, beta):
    a, b, cnt, t, slots, label = _rows()[case]
    da, db, _, _ = _dense(a, b, cnt, t, slots)
    g = -0.625
    rep = lambda v: np.repeat(np.asarray(v, dtype=np.float64), cnt)
    label = "%s jsd beta=%g" % (label, beta)
    v, _ = Gr.jsd_fwd(a, b, cnt, beta)
    _close(v, J.jsd_fwd(da, db, beta)[0][0], label + " fwd", J.cond_jsd_fwd(da, db, beta)[0])
    gs, gt = Gr.jsd_bwd(a, b, cnt, g, beta)
    rs, rt = J.jsd_bwd(da, db, [g], beta)
    cs, ct = J.cond_jsd_bwd(da, db, [g], beta)
    _close(rep(gs), rs[0], label + " bwd s", cs[0])
    _close(rep(gt), rt[0], label + " bwd t", ct[0])
    if np.isfinite(v):
        _close(Gr.cond_jsd_fwd(a, b, cnt, beta), J.cond_jsd_fwd(da, db, beta)[0], label + " cond fwd")
        gcs, gct = Gr.cond_jsd_bwd(a, b, cnt, g, beta)
        _close(rep(gcs), cs[0], label + " cond bwd s")
        _close(rep(gct), ct[0], label + " cond bwd t")


def test_grouped_rejects_shared_target_group():
    with pytest.raises(ValueError):
        Gr.logprobs_fwd(np.array([0.0, 1.0]), np.array([3, 2]), 0)
    with pytest.raises(ValueError):
        Gr.log_softmax(np.array([0.0]), np.array([0]))


def test_pins_catch_planted_mistakes(monkeypatch):
    """A grouped form that drops the count weights, or flips the sign of the gradient for B,
    must fail the comparison with the dense definitions."""
    orig_lsm, orig_kl = Gr.log_softmax, Gr.kl_bwd
    monkeypatch.setattr(Gr, "log_softmax", lambda z, cnt: orig_lsm(z, np.ones_like(np.asarray(cnt))))
    with pytest.raises(AssertionError):
        test_grouped_matches_dense(0)
    monkeypatch.setattr(Gr, "log_softmax", orig_lsm)

    def flipped(a, b, cnt, g):
        da, db = orig_kl(a, b, cnt, g)
        return da, -db

    monkeypatch.setattr(Gr, "kl_bwd", flipped)
    with pytest.raises(AssertionError):
        test_grouped_matches_dense(1)
