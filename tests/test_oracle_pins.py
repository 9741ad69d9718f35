"""Pins of the fp64 oracle against things other than itself (CPU only).

* 50-digit brute force (tests/mp_reference.py) for values and gradients,
* torch.log_softmax / logsumexp in float64 (a library routine),
* closed forms (uniform and two-level rows, KL(A||A) = 0, masked-uniform KL),
* the single-read identities of PR #8838 (H = log S - W/S,
  KL = W/S_A - log S_A + log S_B), KL >= 0, zero-sum gradient rows,
* the extreme-range and support-mismatch cases the pages describe
  (tests/golden/*.json, each with its citation),
* a +1e4 offset that must not change the result (no cancellation),
* planted mistakes in copies of the oracle that these pins must catch.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import mp_reference as mpr
from oracle import compare, linear_logp, reductions as R

NINF = -np.inf
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_rows(seed=0):
    """Small rows with the structures the pages test: plain, masked, offset, target on a mask."""
    rng = np.random.default_rng(seed)
    rows = []
    rows.append(rng.normal(0, 2, 9))
    r = rng.normal(0, 3, 11)
    r[[2, 7]] = NINF
    rows.append(r)
    rows.append(rng.normal(0, 2, 8) + 1e4)
    r = rng.normal(0, 1, 10)
    r[0] = 25.0  # one dominant entry, others tiny
    rows.append(r)
    r = rng.normal(0, 2, 12)
    r[[0, 5, 11]] = NINF
    rows.append(r)
    return rows


def _rel_close(x, y, tol):
    if math.isinf(y) or math.isnan(y):
        return (math.isnan(x) and math.isnan(y)) or x == y
    return abs(x - y) <= tol * max(1.0, abs(y))


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", [0, 1])
def test_forward_values_match_50_digit_brute_force(seed):
    for z in _tiny_rows(seed):
        V = len(z)
        Z = z[None, :]
        H, _, _ = R.entropy_fwd(Z)
        assert _rel_close(H[0], float(mpr.entropy(list(z))), 1e-13)
        for t in range(V):
            lp, _, _ = R.logprobs_fwd(Z, [t])
            want = mpr.to_float(mpr.logprob(list(z), t))
            if z[t] == NINF:
                assert lp[0] == -np.inf
            else:
                assert _rel_close(lp[0], want, 1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_kl_values_match_50_digit_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    for a in _tiny_rows(seed):
        b = a + rng.normal(0, 0.7, a.shape)
        b[a == NINF] = NINF
        b[rng.integers(0, len(a))] += 1.0
        kl, _ = R.kl_fwd(a[None], b[None])
        assert _rel_close(kl[0], float(mpr.kl(list(a), list(b))), 1e-12)
        # and the other direction
        kl2, _ = R.kl_fwd(b[None], a[None])
        assert _rel_close(kl2[0], float(mpr.kl(list(b), list(a))), 1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_50_digit_differences(seed):
    rng = np.random.default_rng(200 + seed)
    for z in _tiny_rows(seed):
        V = len(z)
        g = rng.normal()
        Z = z[None]
        dH = R.entropy_bwd(Z, [g])[0]
        want = [g * float(v) for v in mpr.entropy_grad(list(z))]
        np.testing.assert_allclose(dH, want, rtol=1e-10, atol=1e-12 * abs(g))
        t = int(rng.integers(0, V))
        while z[t] == NINF:
            t = int(rng.integers(0, V))
        dL = R.logprobs_bwd(Z, [t], [g])[0]
        want = [g * float(v) for v in mpr.logprob_grad(list(z), t)]
        np.testing.assert_allclose(dL, want, rtol=1e-10, atol=1e-12 * abs(g))
        b = z + rng.normal(0, 0.5, z.shape)
        b[z == NINF] = NINF
        da, db = R.kl_bwd(Z, b[None], [g])
        wa, wb = mpr.kl_grads(list(z), list(b))
        np.testing.assert_allclose(da[0], [g * float(v) for v in wa], rtol=1e-9, atol=1e-12 * abs(g))
        np.testing.assert_allclose(db[0], [g * float(v) for v in wb], rtol=1e-9, atol=1e-12 * abs(g))


# -------------------------------------------------------------- library routine

def test_log_softmax_matches_torch_float64():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3, (16, 300))
    z[3, :50] = NINF
    z[4] += 1e4
    lp, m, logS = R.log_softmax_rows(z)
    tz = torch.from_numpy(z)
    ref = torch.log_softmax(tz, dim=1).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_allclose(lp[fin], ref[fin], rtol=1e-13, atol=1e-12)
    assert np.array_equal(np.isneginf(lp), np.isneginf(ref))
    np.testing.assert_allclose(m + logS, torch.logsumexp(tz, dim=1).numpy(), rtol=1e-15)


# ------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("V,offset", [(7, 0.0), (1000, 1e4), (75968, 9984.0), (1, -3.0)])
def test_uniform_row_closed_form(V, offset):
    z = np.full((1, V), offset)
    H, _, _ = R.entropy_fwd(z)
    assert H[0] == pytest.approx(math.log(V), rel=1e-14, abs=1e-15)
    lp, _, _ = R.logprobs_fwd(z, [V // 2])
    assert lp[0] == pytest.approx(-math.log(V), rel=1e-14)
    dH = R.entropy_bwd(z, [1.7])
    assert np.max(np.abs(dH)) <= 1e-15 * max(1.0, math.log(V))
    dL = R.logprobs_bwd(z, [V // 2], [0.5])[0]
    want = -0.5 / V * np.ones(V)
    want[V // 2] += 0.5
    np.testing.assert_allclose(dL, want, rtol=1e-12, atol=1e-18)


def test_two_level_rows_closed_form():
    # k entries at x + d, V - k at x: p_hi = e^d / (k e^d + V - k)
    V, k, d = 50, 3, 2.5
    z = np.zeros((1, V))
    z[0, :k] = d
    Z = k * math.exp(d) + (V - k)
    ph, pl = math.exp(d) / Z, 1.0 / Z
    H = -(k * ph * math.log(ph) + (V - k) * pl * math.log(pl))
    assert R.entropy_fwd(z)[0][0] == pytest.approx(H, rel=1e-14)
    # KL between two two-level rows on the same split
    d2 = -1.0
    b = np.zeros((1, V))
    b[0, :k] = d2
    Z2 = k * math.exp(d2) + (V - k)
    qh, ql = math.exp(d2) / Z2, 1.0 / Z2
    kl = k * ph * math.log(ph / qh) + (V - k) * pl * math.log(pl / ql)
    assert R.kl_fwd(z, b)[0][0] == pytest.approx(kl, rel=1e-13)


def test_kl_of_a_row_with_itself_and_shifted_copy_is_zero():
    rng = np.random.default_rng(9)
    a = np.round(rng.normal(0, 3, (8, 500)) * 64) / 64  # grid values: +c below is exact
    assert np.all(R.kl_fwd(a, a)[0] == 0.0)
    kl, _ = R.kl_fwd(a, a + 1024.0)
    assert np.max(np.abs(kl)) < 1e-12
    da, db = R.kl_bwd(a, a, np.ones(8))
    assert np.max(np.abs(da)) == 0.0 and np.max(np.abs(db)) == 0.0


def test_masked_uniform_kl_closed_forms():
    # A uniform on V; B uniform on V - 64 columns (64 masked): KL(B||A) = log(V/(V-64)); KL(A||B) = +inf
    V = 75968
    a = np.full((1, V), 9984.0)
    b = a.copy()
    b[0, :64] = NINF
    assert R.kl_fwd(b, a)[0][0] == pytest.approx(math.log(V / (V - 64)), rel=1e-12)
    assert R.kl_fwd(a, b)[0][0] == np.inf


# ------------------------------------------------------------------- identities

def test_single_read_identities_and_invariants():
    rng = np.random.default_rng(11)
    a = rng.normal(0, 3, (12, 2000))
    b = a + rng.normal(0, 0.5, a.shape)
    a[2] += 1e4
    b[2] += 1e4
    a[5, :100] = NINF
    b[5, :100] = NINF
    H, _, _ = R.entropy_fwd(a)
    H2, KL2 = R.single_read_identities(a, b)
    np.testing.assert_allclose(H, H2, rtol=1e-11)
    kl, _ = R.kl_fwd(a, b)
    np.testing.assert_allclose(kl, KL2, rtol=1e-9, atol=1e-12)
    assert np.all(kl >= 0)
    g = rng.normal(size=12)
    for grad in (R.entropy_bwd(a, g), R.logprobs_bwd(a, rng.integers(100, 2000, 12), g), *R.kl_bwd(a, b, g)):
        np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-12 * max(1.0, np.abs(grad).max()))


def test_large_offset_does_not_cancel():
    # z + 1e4 is exact in float64 for these fp32 values, so every result must be unchanged
    rng = np.random.default_rng(13)
    z = rng.normal(0, 2, (4, 1024)).astype(np.float32).astype(np.float64)
    zo = z + 1e4
    np.testing.assert_allclose(R.entropy_fwd(zo)[0], R.entropy_fwd(z)[0], rtol=1e-12)
    t = rng.integers(0, 1024, 4)
    np.testing.assert_allclose(R.logprobs_fwd(zo, t)[0], R.logprobs_fwd(z, t)[0], rtol=1e-12)
    b = z + rng.normal(0, 0.5, z.shape)
    np.testing.assert_allclose(R.kl_fwd(zo, b + 1e4)[0], R.kl_fwd(z, b)[0], rtol=1e-9)
    np.testing.assert_allclose(R.entropy_bwd(zo, np.ones(4)), R.entropy_bwd(z, np.ones(4)), rtol=1e-9, atol=1e-15)


# ------------------------------------------------------- the pages' special cases

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_extreme_range_rows():
    gold = _load("extreme_range.json")
    for case in gold["cases"]:
        z = np.array([[float(v) for v in case["row"]]])
        H, _, _ = R.entropy_fwd(z)
        assert H[0] == case["entropy"]
        assert R.kl_fwd(z, z)[0][0] == case["kl_self"]
        assert np.all(R.entropy_bwd(z, [1.0]) == 0.0)
        da, db = R.kl_bwd(z, z, [1.0])
        assert np.all(da == 0.0) and np.all(db == 0.0)


def test_golden_support_mismatch():
    gold = _load("support_mismatch.json")
    for case in gold["cases"]:
        a = np.array([[float(v) for v in case["a"]]])
        b = np.array([[float(v) for v in case["b"]]])
        kl, _ = R.kl_fwd(a, b)
        assert kl[0] == float(case["kl"])
        if case["kl"] == "inf":
            da, db = R.kl_bwd(a, b, [1.0])
            assert np.all(np.isnan(da)) and np.all(np.isfinite(db))


def test_undefined_rows_and_targets():
    z = np.array([[NINF, NINF, NINF], [0.0, np.nan, 1.0], [0.0, np.inf, 1.0], [0.0, 1.0, 2.0]])
    H, _, _ = R.entropy_fwd(z)
    assert np.all(np.isnan(H[:3])) and np.isfinite(H[3])
    lp, _, _ = R.logprobs_fwd(z, [0, 0, 0, 5], ignore_index=-100)
    assert np.all(np.isnan(lp))  # undefined rows and an out-of-range target
    lp, _, _ = R.logprobs_fwd(z, [-100, -100, -100, -100], ignore_index=-100)
    assert np.all(lp == 0)
    d = R.logprobs_bwd(z, [-100, 0, 0, 3], [1.0, 1.0, 1.0, 1.0])
    assert np.all(d[0] == 0) and np.all(np.isnan(d[1:]))
    # KL: A all -inf -> NaN; B all -inf with A live -> +inf
    a = np.array([[NINF, NINF], [0.0, 1.0]])
    b = np.array([[0.0, 1.0], [NINF, NINF]])
    kl, _ = R.kl_fwd(a, b)
    assert np.isnan(kl[0]) and kl[1] == np.inf


# ------------------------------------------------------------------ linear logp

def test_linear_logp_gradients_match_differences():
    rng = np.random.default_rng(21)
    n, k, V = 3, 5, 7
    h = rng.normal(size=(n, k))
    W = rng.normal(0, 0.5, (V, k))
    t = np.array([1, 6, 0])
    g = rng.normal(size=n)

    def loss(hh, WW):
        return float(np.sum(g * linear_logp.linear_logp_fwd(hh, WW, t)[0]))

    eps = 1e-6
    dh = linear_logp.linear_logp_bwd_dh(h, W, t, g)
    dW = linear_logp.linear_logp_bwd_dw(h, W, t, g, row_chunk=2)
    for i in range(n):
        for j in range(k):
            hp, hm = h.copy(), h.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            assert dh[i, j] == pytest.approx((loss(hp, W) - loss(hm, W)) / (2 * eps), rel=1e-6, abs=1e-9)
    for v in range(V):
        for j in range(k):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, j] += eps
            Wm[v, j] -= eps
            assert dW[v, j] == pytest.approx((loss(h, Wp) - loss(h, Wm)) / (2 * eps), rel=1e-6, abs=1e-9)
    # sampled rows / vocab rows agree with the full evaluation
    np.testing.assert_allclose(linear_logp.linear_logp_bwd_dh(h, W, t, g, rows=[2, 0]), dh[[2, 0]])
    np.testing.assert_allclose(linear_logp.linear_logp_bwd_dw(h, W, t, g, vocab_rows=[6, 1]), dW[[6, 1]])
    dw2, c2 = linear_logp.linear_logp_bwd_dw_cond(h, W, t, g, vocab_rows=[6, 1], row_chunk=2)
    np.testing.assert_allclose(dw2, dW[[6, 1]])
    np.testing.assert_allclose(c2, linear_logp.cond_linear_dw(h, W, t, g, vocab_rows=[6, 1]))
    assert np.all(c2 >= np.abs(dw2) - 1e-12)


def test_linear_logp_forward_matches_brute_force():
    rng = np.random.default_rng(22)
    h = rng.normal(size=(2, 6))
    W = rng.normal(0, 0.3, (9, 6))
    t = [4, 8]
    lp, m, logS = linear_logp.linear_logp_fwd(h, W, t)
    for i in range(2):
        z = [float(mpr.mp.fsum(mpr.mp.mpf(h[i, j]) * mpr.mp.mpf(W[v, j]) for j in range(6))) for v in range(9)]
        assert lp[i] == pytest.approx(float(mpr.logprob(z, t[i])), rel=1e-13)


# ------------------------------------------------------------ comparison helpers

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.normal(0, 1, 10000), rng.normal(0, 1e30, 100), rng.normal(0, 1e-30, 100),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.3895e38, 1e-40, 0.0]]).astype(np.float32)
    mine = compare.bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)
    assert compare.bf16_rne(np.array([1 + 2 ** -8]))[0] == 1.0  # tie to even
    assert compare.bf16_rne(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_f16_rne_matches_torch_and_numpy_casts():
    rng = np.random.default_rng(32)
    x = np.concatenate([rng.normal(0, 1, 10000), rng.normal(0, 3e4, 200), rng.normal(0, 1e-6, 200),
                        rng.normal(0, 1e-9, 50), [1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 65519.0, 65520.0,
                                                  2 ** -25, 3 * 2 ** -26, 0.0]])
    mine = compare.f16_rne(x)
    ref_np = x.astype(np.float16).astype(np.float64)
    ref_torch = torch.from_numpy(x.astype(np.float32)).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref_np)
    exact32 = x.astype(np.float32).astype(np.float64) == x  # values a float32 holds exactly: no double rounding
    np.testing.assert_array_equal(mine[exact32], ref_torch[exact32])
    assert compare.f16_rne(np.array([1 + 2 ** -11]))[0] == 1.0  # tie to even
    assert compare.f16_rne(np.array([65520.0]))[0] == np.inf
    assert compare.ulp_f16(np.array([1.0, 2 ** -20, 0.0]))[0] == 2 ** -10
    assert compare.ulp_f16(np.array([2 ** -20]))[0] == 2 ** -24


def test_check_accepts_exact_and_rejects_planted_errors():
    y = np.array([1.0, -2.5, 1e-3, np.inf, np.nan])
    c = np.abs(y)
    assert compare.check(y.astype(np.float32), y, c, "f32")["fail"] == 0
    bad = y.copy()
    bad[0] *= 1 + 1e-4
    assert compare.check(bad, y, c, "f32")["fail"] == 1
    bad = y.copy()
    bad[3] = 1.0
    r = compare.check(bad, y, c, "f32")
    assert r["inf_mismatch"] == 1
    bad = y.copy()
    bad[4] = 0.0
    assert compare.check(bad, y, c, "f32")["nan_mismatch"] == 1
    yb = compare.bf16_rne(np.array([1.0, 3.0, -0.75]))
    assert compare.check(yb, yb, np.zeros(3), "bf16")["fail"] == 0
    off2 = yb + 2 * compare.ulp_bf16(yb)
    assert compare.check(off2, yb, np.zeros(3), "bf16")["fail"] == 3


def test_check_reports_max_relative_error_of_fp32_values():
    """max_rel is the largest |x - y| / |y| over finite nonzero y; zeros, inf and NaN take no part."""
    y = np.array([2.0, -4.0, 0.0, np.inf, np.nan, 0.5])
    x = y.copy()
    x[0] = 2.0 * (1 + 3e-7)
    x[1] = -4.0 * (1 - 1e-6)
    x[2] = 1e-30
    x[5] = 0.5 * (1 + 2e-7)
    r = compare.check(x, y, np.abs(np.nan_to_num(y, posinf=0.0)), "f32")
    assert abs(r["max_rel"] - 1e-6) < 1e-12
    assert compare.check(y, y, np.zeros(6), "f32")["max_rel"] == 0.0
    assert compare.check(np.zeros(2), np.zeros(2), np.zeros(2), "f32")["max_rel"] == 0.0
    yb = compare.bf16_rne(np.array([1.0, 3.0]))
    assert compare.check(yb, yb, np.zeros(2), "bf16")["max_rel"] is None


# ------------------------------------------------------ planted-mistake detection

def _entropy_bwd_dropped_H(z, g):
    lp, _, _ = R.log_softmax_rows(z)
    p = np.exp(lp)
    return np.where(z > -np.inf, -np.asarray(g)[:, None] * p * lp, 0.0)


def _kl_bwd_wrong_sign_b(a, b, g):
    da, db = R.kl_bwd(a, b, g)
    return da, -db


def _logprobs_bwd_no_onehot(z, t, g):
    lp, _, _ = R.log_softmax_rows(z)
    return -np.asarray(g)[:, None] * np.exp(lp)


def test_pins_catch_planted_mistakes():
    """Each mutant of the oracle must fail at least one pin above."""
    z = _tiny_rows(0)[1]
    g = 0.7
    want_H = [g * float(v) for v in mpr.entropy_grad(list(z))]
    assert not np.allclose(_entropy_bwd_dropped_H(z[None], [g])[0], want_H, rtol=1e-6)
    b = z + 0.3
    b[z == NINF] = NINF
    b[0] += 1.0
    wa, wb = mpr.kl_grads(list(z), list(b))
    assert not np.allclose(_kl_bwd_wrong_sign_b(z[None], b[None], [g])[1][0], [g * float(v) for v in wb], rtol=1e-6)
    t = 3
    wl = [g * float(v) for v in mpr.logprob_grad(list(z), t)]
    assert not np.allclose(_logprobs_bwd_no_onehot(z[None], [t], [g])[0], wl, rtol=1e-6)
    # a transposed operand in the fused variant breaks the difference pin
    rng = np.random.default_rng(3)
    h = rng.normal(size=(4, 4))
    W = rng.normal(size=(4, 4))
    tt = np.array([0, 1, 2, 3])
    gg = np.ones(4)
    dh = linear_logp.linear_logp_bwd_dh(h, W, tt, gg)
    dh_wrong = R.logprobs_bwd(h @ W.T, tt, gg) @ W.T
    assert not np.allclose(dh, dh_wrong)


# ------------------------------------------------------ rounding-scale pins

def test_condition_scales_closed_forms():
    """The rounding scales of the parity rule on rows where every term is known by hand:
    a uniform row (p = 1/V, z - m = 0, log S = log V, H = log V) and a two-level row."""
    V, off, t = 7, 5.0, 3
    z = np.full((1, V), off)
    g = np.array([-2.0])
    L = np.log(V)
    assert np.isclose(R.cond_logprobs_fwd(z, np.array([t]))[0], L)
    assert np.isclose(R.cond_entropy_fwd(z)[0], L)
    assert np.isclose(R.cond_kl_fwd(z, z)[0], 2 * L)
    cl = R.cond_logprobs_bwd(z, np.array([t]), g)[0]
    want = 2.0 * (np.eye(V)[t] + (1.0 + L) / V)
    np.testing.assert_allclose(cl, want, rtol=1e-13)
    np.testing.assert_allclose(R.cond_entropy_bwd(z, g)[0], 2.0 * (1.0 + 2 * L) / V, rtol=1e-13)
    ca, cb = R.cond_kl_bwd(z, z, g)
    np.testing.assert_allclose(ca[0], 2.0 * (1.0 + 2 * L) / V, rtol=1e-13)
    np.testing.assert_allclose(cb[0], 2.0 * 2 * (1.0 + L) / V, rtol=1e-13)
    # two levels: z = (0, -1): m = 0, p = (1, e^-1) / (1 + e^-1), |z - m| = (0, 1)
    z2 = np.array([[0.0, -1.0]])
    S = 1.0 + np.exp(-1.0)
    p1 = np.exp(-1.0) / S
    assert np.isclose(R.cond_entropy_fwd(z2)[0], np.log(S) + p1)
    assert np.isclose(R.cond_logprobs_fwd(z2, np.array([1]))[0], 1.0 + np.log(S))
    # a KL pair with KL != 0: a = (0, -1), b = (-1, 0); both have log S = log(1 + e^-1),
    # p_A = (1, e^-1) / S, p_B = (e^-1, 1) / S, KL = (1 - e^-1) / S
    a2, b2 = np.array([[0.0, -1.0]]), np.array([[-1.0, 0.0]])
    lS = np.log(S)
    pa = np.array([1.0, np.exp(-1.0)]) / S
    pb = pa[::-1]
    kl = (1.0 - np.exp(-1.0)) / S
    assert np.isclose(R.kl_fwd(a2, b2)[0][0], kl)
    assert np.isclose(R.cond_kl_fwd(a2, b2)[0], 1.0 + 2 * lS)
    ca, cb = R.cond_kl_bwd(a2, b2, np.array([0.5]))
    np.testing.assert_allclose(ca[0], 0.5 * pa * (2.0 + 2 * lS + kl), rtol=1e-13)
    np.testing.assert_allclose(cb[0], 0.5 * (pa * (1.0 + np.array([0.0, 1.0]) + lS) +
                                             pb * (1.0 + np.array([1.0, 0.0]) + lS)), rtol=1e-13)
    # masked entries add nothing
    z3 = np.array([[0.0, -1.0, -np.inf]])
    assert np.isclose(R.cond_entropy_fwd(z3)[0], np.log(S) + p1)
    assert R.cond_entropy_bwd(z3, np.array([1.0]))[0, 2] == 0.0


def test_condition_scales_keep_the_rule_tight():
    """On realistic rows the rounding allowance stays far below the errors a wrong kernel
    makes: every forward value off by 0.2% of max(|y|, 1) (KL near 0 is a difference of
    terms of size log S, so its allowance is absolute) is rejected, the scales stay of the
    order of log V, and a bf16 gradient entry off by 2 ulps is rejected wherever the
    computation is not near a cancellation."""
    rng = np.random.default_rng(11)
    n, V = 16, 3000
    a = 3.0 * rng.standard_normal((n, V))
    b = a + 0.5 * rng.standard_normal((n, V))
    a[0] += 1e4
    b[0] += 1e4
    t = rng.integers(0, V, n)
    g = rng.standard_normal(n)
    cases = [
        (R.logprobs_fwd(a, t)[0], R.cond_logprobs_fwd(a, t)),
        (R.entropy_fwd(a)[0], R.cond_entropy_fwd(a)),
        (R.kl_fwd(a, b)[0], R.cond_kl_fwd(a, b)),
    ]
    for y, c in cases:
        assert compare.check(y, y, c, "f32")["fail"] == 0
        assert np.all(c < 4 * (np.log(V) + 30.0))
        off = y + 2e-3 * np.maximum(np.abs(y), 1.0)
        assert compare.check(off, y, c, "f32")["fail"] == n
    # (gradient, scale, largest share of entries near a cancellation): the KL gradient
    # w.r.t. A cancels wherever log p_A - log p_B is close to KL, which for B = A + noise is
    # common, so only the logprobs and entropy shares are bounded
    grads = [
        (R.logprobs_bwd(a, t, g), R.cond_logprobs_bwd(a, t, g), 0.0),
        (R.entropy_bwd(a, g), R.cond_entropy_bwd(a, g), 1e-3),
        (R.kl_bwd(a, b, g)[0], R.cond_kl_bwd(a, b, g)[0], 1.0),
        (R.kl_bwd(a, b, g)[1], R.cond_kl_bwd(a, b, g)[1], 1.0),
    ]
    for y, c, share in grads:
        yb = compare.bf16_rne(y)
        assert compare.check(yb, y, c, "bf16")["fail"] == 0
        u = compare.ulp_bf16(yb)
        live = np.abs(yb) > 1e-30
        # entries near a cancellation may carry more than half an ulp of fp32 rounding;
        # every other entry is held to one ulp
        loose = live & (compare.COND * c >= 0.5 * u)  # 2 ulps off rne(y) is >= 1.5 ulps off y
        assert loose.sum() <= share * live.sum()
        tight = live & ~loose
        off = np.where(live, yb + 2 * u * np.sign(yb), yb)
        assert compare.check(off[tight], y[tight], c[tight], "bf16")["fail"] == int(tight.sum())


def test_condition_scales_of_topk_jsd_and_linear():
    """The rounding scales of the other oracles: top-k with one slot reduces to the single-id
    scales and a duplicated id adds the slots' |g|; the JSD scales on an identical uniform
    pair and their KL endpoints; the linear-logp scales on constant logits."""
    from oracle import jsd as J, topk as TK

    rng = np.random.default_rng(4)
    z = 2.0 * rng.standard_normal((5, 40))
    t = rng.integers(0, 40, 5)
    g = rng.standard_normal(5)
    np.testing.assert_allclose(TK.cond_logprobs_topk_fwd(z, t[:, None])[:, 0], R.cond_logprobs_fwd(z, t))
    np.testing.assert_allclose(TK.cond_logprobs_topk_bwd(z, t[:, None], g[:, None]), R.cond_logprobs_bwd(z, t, g))
    ids = np.stack([t, t], axis=1)
    gg = np.stack([g, -0.5 * g], axis=1)
    c2 = TK.cond_logprobs_topk_bwd(z, ids, gg)
    c1 = R.cond_logprobs_bwd(z, t, 1.5 * np.abs(g))
    np.testing.assert_allclose(c2, c1)  # |g1| + |g2| on the one-hot and on the softmax part
    # JSD on s = t uniform over V: p = 1/V, log p = log M = -log V, no centring term, K = 0
    V, beta = 9, 0.3
    L = np.log(V)
    u = np.zeros((1, V))
    assert np.isclose(J.cond_jsd_fwd(u, u, beta)[0], 6 * L)
    cs, ct = J.cond_jsd_bwd(u, u, np.array([2.0]), beta)
    np.testing.assert_allclose(cs[0], 2.0 * (1 - beta) * (1 + 3 * L) / V, rtol=1e-13)
    np.testing.assert_allclose(ct[0], 2.0 * beta * (1 + 3 * L) / V, rtol=1e-13)
    np.testing.assert_allclose(J.cond_jsd_fwd(z, z[::-1], 0.0), R.cond_kl_fwd(z[::-1], z))
    np.testing.assert_allclose(J.cond_jsd_fwd(z, z[::-1], 1.0), R.cond_kl_fwd(z, z[::-1]))
    ks, kt = J.cond_jsd_bwd(z, z[::-1], g, 0.0)
    rt, rs = R.cond_kl_bwd(z[::-1], z, g)
    np.testing.assert_allclose(ks, rs)
    np.testing.assert_allclose(kt, rt)
    # linear-logp: W a column of ones (H = 1) makes every logit of token n equal to h_n
    n, Vl = 4, 6
    h = rng.standard_normal((n, 1))
    W = np.ones((Vl, 1))
    tl = np.array([0, 5, 2, -100])
    gl = np.array([1.0, -2.0, 0.5, 3.0])
    np.testing.assert_allclose(linear_logp.cond_logits(np.abs(h), W), np.abs(h) @ W.T)
    cf = linear_logp.cond_linear_fwd(h, W, tl)
    # |z_t - m| = 0, |log S| = log V, cz = |h_n| for every v, sum_v p_v cz_v = |h_n|
    np.testing.assert_allclose(cf[:3], np.log(Vl) + 2 * np.abs(h[:3, 0]), rtol=1e-13)
    np.testing.assert_allclose(cf[3], np.log(Vl) + np.abs(h[3, 0]), rtol=1e-13)
    # dz = g (1[v = t] - 1/V): sum_v |dz_v| = 2 |g| (1 - 1/V); an ignored token adds nothing
    cdh = linear_logp.cond_linear_dh(h, W, tl, gl)[:, 0]
    np.testing.assert_allclose(cdh[:3], 2 * np.abs(gl[:3]) * (1 - 1 / Vl), rtol=1e-13)
    assert cdh[3] == 0.0
    # dz scale: the logits-op scale |g| (1[v = t] + (1 + log V) / V) plus |g| (cz + sum p cz) / V
    cdz = linear_logp.cond_linear_dz(h, W, tl, gl)
    one = np.zeros((n, Vl))
    one[np.arange(3), tl[:3]] = 1.0
    want_dz = np.abs(gl)[:, None] * (one + (1 + np.log(Vl) + 2 * np.abs(h)) / Vl)
    np.testing.assert_allclose(cdz[:3], want_dz[:3], rtol=1e-13)
    np.testing.assert_allclose(cdz[3], np.abs(gl[3]) * (1 + np.log(Vl)) / Vl, rtol=1e-13)  # ignored: no logit term
    dz = linear_logp.linear_logp_bwd_dz(h, W, tl, gl)
    np.testing.assert_allclose(dz[:3], gl[:3, None] * (one[:3] - 1.0 / Vl), rtol=1e-13)
    cdw = linear_logp.cond_linear_dw(h, W, tl, gl)[:, 0]
    want = np.zeros(Vl)
    for i in range(3):
        want += np.abs(gl[i]) * np.abs(h[i, 0]) * np.where(np.arange(Vl) == tl[i], 1 - 1 / Vl, 1 / Vl)
    np.testing.assert_allclose(cdw, want, rtol=1e-13)
