"""Pins of the generalized JSD oracle against things other than itself (CPU only).

* scipy.spatial.distance.jensenshannon (natural log) squared equals JSD at beta = 0.5;
* torch float64 autograd of the definition gives the closed-form gradients;
* 50-digit brute force (mpmath) of the definition for values, central
  differences for gradients, at interior beta, with masked columns and a +1e4 row;
* closed forms: disjoint supports give the binary entropy of beta; JSD(P, P) = 0
  with zero gradients; JSD_beta(S, T) = JSD_(1-beta)(T, S);
* the endpoint branches are the KL oracle (beta = 0: KL(T||S), beta = 1: KL(S||T));
* the convention of the mixture: as beta -> 0 the student gradient divided by
  beta tends to the forward-KL gradient p_S - p_T, and as beta -> 1 the teacher
  gradient divided by (1 - beta) tends to the reverse-KL gradient p_T - p_S
  (GKD-style generalized JSD, mixture weight beta on the teacher);
* planted mistakes (mixture weights swapped, the K_S term dropped from the
  gradient) that these pins catch.
"""

import math

import mpmath as mp
import numpy as np
import pytest
import torch
from scipy.spatial.distance import jensenshannon

from oracle import jsd as J, reductions as R

NINF = -np.inf
mp.mp.dps = 50


def _rows(seed, n=4, v=11, masked=True):
    rng = np.random.default_rng(seed)
    s = rng.normal(0, 2.0, (n, v))
    t = s + rng.normal(0, 1.0, (n, v))
    if masked:
        s[1, [2, 5]] = NINF
        t[2, [0, 3]] = NINF
        s[3] += 1e4
        t[3] += 1e4
    return s, t


def _mp_jsd(s, t, beta):
    """Definition at 50 digits: M = (1 - beta) p_S + beta p_T, beta KL(T||M) + (1 - beta) KL(S||M)."""
    b = mp.mpf(beta)

    def probs(z):
        e = [mp.e ** mp.mpf(x) if x != NINF else mp.mpf(0) for x in z]
        tot = mp.fsum(e)
        return [x / tot for x in e]

    ps, pt = probs(s), probs(t)
    tot = mp.mpf(0)
    for a, c in zip(ps, pt):
        m = (1 - b) * a + b * c
        if c > 0:
            tot += b * c * mp.log(c / m)
        if a > 0:
            tot += (1 - b) * a * mp.log(a / m)
    return tot


def _mp_grad(f, z, step=mp.mpf("1e-22")):
    out = []
    for j, x in enumerate(z):
        if x == NINF:
            out.append(mp.mpf(0))
            continue
        zp, zm = list(map(mp.mpf, z)), list(map(mp.mpf, z))
        zp[j] += step
        zm[j] -= step
        out.append((f(zp) - f(zm)) / (2 * step))
    return out


def _mpify(z):
    return [x if x == NINF else mp.mpf(x) for x in z]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_beta_half_matches_scipy_jensenshannon(seed):
    s, t = _rows(seed, masked=False)
    out, _ = J.jsd_fwd(s, t, 0.5)
    for r in range(s.shape[0]):
        ps = np.exp(s[r] - s[r].max())
        pt = np.exp(t[r] - t[r].max())
        ref = jensenshannon(ps / ps.sum(), pt / pt.sum()) ** 2
        assert abs(out[r] - ref) <= 1e-13 * max(1.0, ref)


@pytest.mark.parametrize("beta", [0.3, 0.7])
def test_gradients_match_torch_float64_autograd(beta):
    s, t = _rows(3, masked=False)
    g = np.array([0.5, -1.25, 2.0, 0.75])
    st = torch.tensor(s, requires_grad=True)
    tt = torch.tensor(t, requires_grad=True)
    ls, lt = torch.log_softmax(st, 1), torch.log_softmax(tt, 1)
    lm = torch.log((1 - beta) * ls.exp() + beta * lt.exp())
    val = beta * (lt.exp() * (lt - lm)).sum(1) + (1 - beta) * (ls.exp() * (ls - lm)).sum(1)
    (val * torch.tensor(g)).sum().backward()
    out, _ = J.jsd_fwd(s, t, beta)
    ds, dt = J.jsd_bwd(s, t, g, beta)
    np.testing.assert_allclose(out, val.detach().numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ds, st.grad.numpy(), rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dt, tt.grad.numpy(), rtol=1e-9, atol=1e-14)


@pytest.mark.parametrize("beta", [0.2, 0.5, 0.9])
def test_values_and_gradients_match_50_digit_brute_force(beta):
    s, t = _rows(4, n=4, v=8)
    out, _ = J.jsd_fwd(s, t, beta)
    g = np.array([1.0, -0.5, 2.0, 1.5])
    ds, dt = J.jsd_bwd(s, t, g, beta)
    for r in range(s.shape[0]):
        ref = float(_mp_jsd(_mpify(s[r]), _mpify(t[r]), beta))
        assert abs(out[r] - ref) <= 1e-12 * max(1.0, abs(ref)) + 1e-13, (r, out[r], ref)
        gs = _mp_grad(lambda z, r=r: _mp_jsd(z, _mpify(t[r]), beta), list(s[r]))
        gt = _mp_grad(lambda z, r=r: _mp_jsd(_mpify(s[r]), z, beta), list(t[r]))
        for j in range(s.shape[1]):
            assert abs(ds[r, j] - g[r] * float(gs[j])) <= 1e-10 * max(1.0, abs(g[r] * float(gs[j]))), (r, j)
            assert abs(dt[r, j] - g[r] * float(gt[j])) <= 1e-10 * max(1.0, abs(g[r] * float(gt[j]))), (r, j)


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.8])
def test_disjoint_support_is_binary_entropy(beta):
    s = np.array([[1.0, 2.0, NINF, NINF, 0.5], [NINF, 3.0, NINF, 1.0, NINF]])
    t = np.array([[NINF, NINF, 0.3, 1.7, NINF], [2.0, NINF, 0.0, NINF, -1.0]])
    out, _ = J.jsd_fwd(s, t, beta)
    hb = -beta * math.log(beta) - (1 - beta) * math.log(1 - beta)
    np.testing.assert_allclose(out, hb, rtol=1e-14)
    ds, dt = J.jsd_bwd(s, t, np.ones(2), beta)
    # each side's log-ratio is constant on its support, so its gradient vanishes
    np.testing.assert_allclose(ds, 0.0, atol=1e-15)
    np.testing.assert_allclose(dt, 0.0, atol=1e-15)


def test_identical_inputs_and_swap_symmetry():
    s, t = _rows(5)
    for beta in (0.25, 0.5, 0.6):
        out, _ = J.jsd_fwd(s, s, beta)
        np.testing.assert_allclose(out, 0.0, atol=1e-14)
        ds, dt = J.jsd_bwd(s, s, np.ones(s.shape[0]), beta)
        np.testing.assert_allclose(ds, 0.0, atol=1e-14)
        np.testing.assert_allclose(dt, 0.0, atol=1e-14)
        a, _ = J.jsd_fwd(s, t, beta)
        b, _ = J.jsd_fwd(t, s, 1 - beta)
        np.testing.assert_allclose(a, b, rtol=1e-13)
        assert (a >= -1e-15).all()


def test_endpoints_are_the_kl_branches():
    s, t = _rows(6)
    g = np.linspace(-1, 1, s.shape[0])
    np.testing.assert_array_equal(J.jsd_fwd(s, t, 0.0)[0], R.kl_fwd(t, s)[0])
    np.testing.assert_array_equal(J.jsd_fwd(s, t, 1.0)[0], R.kl_fwd(s, t)[0])
    ds, dt = J.jsd_bwd(s, t, g, 0.0)
    rt, rs = R.kl_bwd(t, s, g)
    np.testing.assert_array_equal(ds, rs)
    np.testing.assert_array_equal(dt, rt)


def test_small_beta_limits_fix_the_mixture_convention():
    s, t = _rows(7, masked=False)
    ps = np.exp(R.log_softmax_rows(s)[0])
    pt = np.exp(R.log_softmax_rows(t)[0])
    g = np.ones(s.shape[0])
    eps = 1e-6
    ds, _ = J.jsd_bwd(s, t, g, eps)
    np.testing.assert_allclose(ds / eps, ps - pt, rtol=1e-4, atol=1e-8)  # forward KL(T||S) gradient
    _, dt = J.jsd_bwd(s, t, g, 1 - eps)
    np.testing.assert_allclose(dt / eps, pt - ps, rtol=1e-4, atol=1e-8)  # reverse KL(S||T) gradient


def test_extreme_range_rows_have_zero_divergence():
    """A row spanning -3e38..3e38 is one-hot in float64 too (the other entries underflow):
    JSD(p, p) = 0 with zero gradients, and against a different one-hot row the binary
    entropy of beta (disjoint supports), as the zero-weight rule requires."""
    v = 12
    s = np.full((2, v), -3e38)
    s[:, 4] = 3e38
    t = s.copy()
    t[1, 4] = -3e38
    t[1, 9] = 3e38
    for beta in (0.2, 0.5):
        out, _ = J.jsd_fwd(s, t, beta)
        ds, dt = J.jsd_bwd(s, t, np.ones(2), beta)
        assert out[0] == 0.0 and (ds[0] == 0).all() and (dt[0] == 0).all()
        hb = -beta * math.log(beta) - (1 - beta) * math.log(1 - beta)
        assert abs(out[1] - hb) < 1e-15
        assert np.isfinite(ds).all() and np.isfinite(dt).all()


def test_undefined_rows_are_nan():
    s, t = _rows(8)
    s[0, 3] = np.nan
    t[1, :] = NINF
    s[2, 4] = np.inf
    out, _ = J.jsd_fwd(s, t, 0.4)
    ds, dt = J.jsd_bwd(s, t, np.ones(s.shape[0]), 0.4)
    assert np.isnan(out[:3]).all() and np.isfinite(out[3])
    assert np.isnan(ds[:3]).all() and np.isnan(dt[:3]).all() and np.isfinite(ds[3]).all()


def _planted_swapped_mixture(s, t, g, beta):
    """Mistake: mixture weight beta on the student instead of the teacher."""
    ls, lt = R.log_softmax_rows(s)[0], R.log_softmax_rows(t)[0]
    ps, pt = np.exp(ls), np.exp(lt)
    lm = np.log(beta * ps + (1 - beta) * pt)
    Ks = np.sum(ps * (ls - lm), axis=1)
    return g[:, None] * (1 - beta) * ps * ((ls - lm) - Ks[:, None])


def _planted_dropped_ks(s, t, g, beta):
    """Mistake: the row term K_S left out of the student gradient."""
    ls, lt = R.log_softmax_rows(s)[0], R.log_softmax_rows(t)[0]
    ps, pt = np.exp(ls), np.exp(lt)
    lm = np.log((1 - beta) * ps + beta * pt)
    return g[:, None] * (1 - beta) * ps * (ls - lm)


def test_pins_catch_planted_mistakes():
    s, t = _rows(9, masked=False)
    g = np.ones(s.shape[0])
    beta = 0.3
    st = torch.tensor(s, requires_grad=True)
    ls, lt = torch.log_softmax(st, 1), torch.log_softmax(torch.tensor(t), 1)
    lm = torch.log((1 - beta) * ls.exp() + beta * lt.exp())
    (beta * (lt.exp() * (lt - lm)).sum() + (1 - beta) * (ls.exp() * (ls - lm)).sum()).backward()
    ref = st.grad.numpy()
    for bad in (_planted_swapped_mixture(s, t, g, beta), _planted_dropped_ks(s, t, g, beta)):
        assert np.max(np.abs(bad - ref)) > 1e-4
    eps = 1e-6
    ps, pt = np.exp(R.log_softmax_rows(s)[0]), np.exp(R.log_softmax_rows(t)[0])
    swapped_small = _planted_swapped_mixture(s, t, g, eps) / eps
    assert np.max(np.abs(swapped_small - (ps - pt))) > 1e-2
