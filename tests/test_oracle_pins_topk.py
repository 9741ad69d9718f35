"""Pins of the multi-id (top-k) logprobs oracle against things other than itself (CPU only).

* torch in float64: log_softmax + gather for the values, autograd of
  sum g * gather(log_softmax(z), ids) for the gradient (a library routine whose
  backward scatter-adds duplicate ids);
* 50-digit brute force (tests/mp_reference.py) for values and, by central
  differences, for the gradient of sum_k g_k logp(id_k) with duplicates;
* closed forms on a uniform row (log p = -log V; dz = count_j g - G / V);
* the cases the pages list: duplicate ids, ignored ids, a fully ignored row;
* a planted mistake (duplicates assigned instead of added) that the pins catch.
"""

import math

import mpmath as mp
import numpy as np
import pytest
import torch

import mp_reference as mpr
from oracle import reductions as R, topk as TK

NINF = -np.inf
IGN = -100


def _case(seed=0, n=6, V=13, K=5):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 2.5, (n, V))
    z[1, [0, 4]] = NINF
    z[2] += 1e4
    ids = rng.integers(0, V, (n, K))
    if K >= 4:
        ids[0, 1] = ids[0, 3]  # duplicate
    if n > 3:
        ids[3, :] = ids[3, 0]  # all slots the same id
    if n > 4 and K >= 3:
        ids[4, 2] = IGN
    if n > 5:
        ids[5, :] = IGN  # fully ignored row
    ids[1, 0] = 0  # an id on a masked column (logp = -inf, finite gradient)
    g = rng.normal(0, 1, (n, K))
    return z, ids, g


def _torch_ref(z, ids, g):
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    idt = torch.tensor(ids)
    live = idt != IGN
    lp = torch.log_softmax(zt, dim=1).gather(1, torch.where(live, idt, 0))
    out = torch.where(live, lp, torch.zeros_like(lp))
    (out * torch.tensor(g) * live).sum().backward()
    return out.detach().numpy(), zt.grad.numpy()


def _close(x, y, tol=1e-12):
    assert x.shape == y.shape
    same_nan = np.isnan(x) == np.isnan(y)
    assert same_nan.all()
    ok = ~np.isnan(y)
    fin = ok & np.isfinite(y)
    assert (x[ok & ~fin] == y[ok & ~fin]).all()
    assert np.all(np.abs(x[fin] - y[fin]) <= tol * np.maximum(1.0, np.abs(y[fin])))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_matches_torch_float64_autograd(seed):
    z, ids, g = _case(seed)
    out, m, ls = TK.logprobs_topk_fwd(z, ids, IGN)
    dz = TK.logprobs_topk_bwd(z, ids, g, IGN)
    ref_out, ref_dz = _torch_ref(z, ids, g)
    _close(out, ref_out)
    _close(dz, ref_dz, 1e-11)
    assert (out[5] == 0).all() and (dz[5] == 0).all()
    assert out[1, 0] == NINF and np.isfinite(dz[1]).all()


@pytest.mark.parametrize("seed", [3, 4])
def test_topk_values_and_gradient_match_50_digit_brute_force(seed):
    z, ids, g = _case(seed, n=4, V=9, K=4)
    # a masked target makes the loss -inf, which has no differences (the torch pin covers it)
    for r in range(ids.shape[0]):
        for k in range(ids.shape[1]):
            if ids[r, k] != IGN and z[r, ids[r, k]] == NINF:
                ids[r, k] = 1
    out, _, _ = TK.logprobs_topk_fwd(z, ids, IGN)
    dz = TK.logprobs_topk_bwd(z, ids, g, IGN)
    for r in range(z.shape[0]):
        zr = list(z[r])
        live = [k for k in range(ids.shape[1]) if ids[r, k] != IGN]
        for k in live:
            ref = float(mpr.logprob(zr, int(ids[r, k])))
            assert out[r, k] == ref or abs(out[r, k] - ref) <= 1e-13 * max(1.0, abs(ref))

        def L(zz, r=r, live=live):
            lp = mpr.logp_row(zz)
            return mp.fsum(mp.mpf(g[r, k]) * lp[int(ids[r, k])] for k in live)

        gr = mpr.grad(L, zr)
        for j in range(z.shape[1]):
            if z[r, j] == NINF:
                continue  # a masked column has no derivative to difference; the torch pin covers it
            ref = float(gr[j])
            assert abs(dz[r, j] - ref) <= 1e-12 * max(1.0, abs(ref)), (r, j, dz[r, j], ref)


def test_topk_uniform_row_closed_form():
    V, K = 17, 6
    z = np.full((1, V), 3.25)
    ids = np.array([[2, 2, 5, IGN, 16, 2]])
    g = np.array([[0.5, -1.25, 2.0, 7.0, 0.75, 1.5]])
    out, _, _ = TK.logprobs_topk_fwd(z, ids, IGN)
    assert np.allclose(out[0, [0, 1, 2, 4, 5]], -math.log(V), rtol=0, atol=1e-15) and out[0, 3] == 0
    dz = TK.logprobs_topk_bwd(z, ids, g, IGN)
    G = 0.5 - 1.25 + 2.0 + 0.75 + 1.5
    want = np.full(V, -G / V)
    want[2] += 0.5 - 1.25 + 1.5
    want[5] += 2.0
    want[16] += 0.75
    assert np.allclose(dz[0], want, rtol=0, atol=1e-15)
    assert abs(dz.sum()) < 1e-14  # gradient rows sum to 0


def test_topk_single_slot_reduces_to_single_id_oracle():
    z, ids, g = _case(7, n=6, V=13, K=1)
    ids[2, 0] = 13  # out of range
    out, m, ls = TK.logprobs_topk_fwd(z, ids, IGN)
    o1, m1, ls1 = R.logprobs_fwd(z, ids[:, 0], IGN)
    np.testing.assert_array_equal(out[:, 0], o1)
    d = TK.logprobs_topk_bwd(z, ids, g, IGN)
    d1 = R.logprobs_bwd(z, ids[:, 0], g[:, 0], IGN)
    np.testing.assert_allclose(d, d1, rtol=1e-14, atol=1e-16)


def test_topk_out_of_range_and_undefined_rows():
    z, ids, g = _case(8)
    ids[0, 2] = -1
    z[3, 4] = np.nan
    ids[4, :] = IGN
    z[4, :] = NINF  # undefined but fully ignored: zeros
    out, _, _ = TK.logprobs_topk_fwd(z, ids, IGN)
    dz = TK.logprobs_topk_bwd(z, ids, g, IGN)
    assert np.isnan(out[0, 2]) and not np.isnan(out[0, [0, 1, 3, 4]]).any()
    assert np.isnan(dz[0]).all()
    assert np.isnan(out[3]).all() and np.isnan(dz[3]).all()
    assert (out[4] == 0).all() and (dz[4] == 0).all()


def _planted_assign_duplicates(z, ids, g):
    """A plausible mistake: scatter by assignment, so a duplicate id keeps only its last g."""
    lp, _, _ = R.log_softmax_rows(z)
    p = np.exp(lp)
    dz = np.zeros_like(z)
    for r in range(z.shape[0]):
        live = ids[r] != IGN
        if not live.any():
            continue
        dz[r, ids[r, live]] = g[r, live]
        dz[r] -= g[r, live].sum() * p[r]
    return dz


def test_pins_catch_planted_duplicate_mistake():
    z, ids, g = _case(0)
    _, ref_dz = _torch_ref(z, ids, g)
    bad = _planted_assign_duplicates(z, ids, g)
    assert np.nanmax(np.abs(bad - ref_dz)) > 1e-3
