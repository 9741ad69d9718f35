"""The parity rule for the fused linear-logp gradients separates an accurate backward from
plausible mistakes (CPU only, no GPU).

RL-Kernel PR #208 ("[Feat][Kernel] Add TP Fused linear logp Triton", review nitpick on the
chunked backward) forms dz = g (onehot(t) - p) in fp32 and contracts it into dh = dz W and
dW = dz^T h. These tests emulate in numpy, on a case whose logit spread matches the fused
workload (h ~ N(0, 1), W scaled so that a logit has standard deviation 1.28, as for
H = 4096 and W ~ N(0, 0.02^2)), the arithmetic of backward designs and hold each to the
standard rule of oracle.compare (no widened factor):

* dz formed in fp32 and contracted with fp32 accumulation: every element passes;
* dz fed as a bf16 pair, hi = rne(dz) and lo = rne(dz - hi), both contracted with fp32
  accumulation (what the HIP backward does): every element passes, worst ratio <= 1;
* dz rounded once to bf16 before the contractions: rejected (entries of dh and dW miss);
* a 2% error on the vocabulary rows of dW that no token targets: rejected;
* dW computed without one 256-token tile: rejected.
"""

import numpy as np
import pytest

from oracle import compare, linear_logp as OL, reductions as R

N, H, V = 1024, 256, 4096


def _bf16(x):
    return compare.bf16_rne(np.asarray(x, dtype=np.float64))


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(2024)
    h = _bf16(rng.standard_normal((N, H)))
    W = _bf16(rng.standard_normal((V, H)) * (1.28 / np.sqrt(H)))
    t = rng.integers(0, V, N)
    t[::61] = -100
    g = rng.standard_normal(N)
    z = OL.logits(h, W)
    dz64 = R.logprobs_bwd(z, t, g)
    # fp32 emulation of the device's dz: fp32 logits (fp32 accumulation), (m, log S) rounded to fp32
    z32 = (h.astype(np.float32) @ W.astype(np.float32).T)
    _, m, ls = R.logprobs_fwd(z, t)
    p32 = np.exp((z32 - m.astype(np.float32)[:, None]) - ls.astype(np.float32)[:, None]).astype(np.float32)
    one = np.zeros_like(p32)
    ok = t >= 0
    one[np.nonzero(ok)[0], t[ok]] = 1.0
    dz32 = (g.astype(np.float32)[:, None] * (one - p32)).astype(np.float32)
    dz32[~ok] = 0.0
    ref = {
        "dh": OL.linear_logp_bwd_dh(h, W, t, g),
        "dh_c": OL.cond_linear_dh(h, W, t, g),
    }
    ref["dW"], ref["dW_c"] = OL.linear_logp_bwd_dw_cond(h, W, t, g)
    return {"h": h, "W": W, "t": t, "g": g, "dz64": dz64, "dz32": dz32, "ref": ref}


def _contract(dz_parts, h, W):
    """dh and dW rounded to bf16, each part contracted with fp32 accumulation and the parts summed in fp32."""
    W32, h32 = W.astype(np.float32), h.astype(np.float32)
    dh = sum(p.astype(np.float32) @ W32 for p in dz_parts)
    dW = sum(p.astype(np.float32).T @ h32 for p in dz_parts)
    return _bf16(dh), _bf16(dW)


def _rep(x, ref, c):
    return compare.check(x, ref, c, "bf16")


def test_accurate_dz_passes(case):
    dh, dW = _contract([case["dz32"]], case["h"], case["W"])
    for name, x in (("dh", dh), ("dW", dW)):
        r = _rep(x, case["ref"][name], case["ref"][name + "_c"])
        assert r["fail"] == 0 and r["nan_mismatch"] == 0 and r["inf_mismatch"] == 0 and r["worst"] <= 1.0, (name, r)


def test_bf16_pair_dz_passes(case):
    hi = _bf16(case["dz32"]).astype(np.float32)
    lo = _bf16(case["dz32"].astype(np.float64) - hi).astype(np.float32)
    # the pair holds dz to about 2^-17 relative
    assert np.all(np.abs((hi.astype(np.float64) + lo) - case["dz32"]) <= 2.0 ** -16 * np.abs(case["dz32"]) + 1e-45)
    dh, dW = _contract([hi, lo], case["h"], case["W"])
    for name, x in (("dh", dh), ("dW", dW)):
        r = _rep(x, case["ref"][name], case["ref"][name + "_c"])
        assert r["fail"] == 0 and r["nan_mismatch"] == 0 and r["inf_mismatch"] == 0 and r["worst"] <= 1.0, (name, r)


def test_single_bf16_dz_is_rejected(case):
    dh, dW = _contract([_bf16(case["dz32"])], case["h"], case["W"])
    rh = _rep(dh, case["ref"]["dh"], case["ref"]["dh_c"])
    rw = _rep(dW, case["ref"]["dW"], case["ref"]["dW_c"])
    assert rh["fail"] > 0.002 * rh["n"], rh
    assert rw["fail"] > 0.002 * rw["n"], rw


def test_two_percent_error_on_untargeted_dw_rows_is_rejected(case):
    dW = case["ref"]["dW"].copy()
    untargeted = np.setdiff1d(np.arange(V), case["t"][case["t"] >= 0])
    dW[untargeted] *= 1.02
    r = _rep(_bf16(dW), case["ref"]["dW"], case["ref"]["dW_c"])
    planted = untargeted.size * H
    assert r["fail"] >= 0.95 * planted, (r, planted)


def test_dropped_token_tile_in_dw_is_rejected(case):
    keep = np.arange(256, N)
    h, t, g = case["h"][keep], case["t"][keep], case["g"][keep]
    dz = R.logprobs_bwd(OL.logits(case["h"], case["W"])[keep], t, g)
    dW = _bf16(dz.T @ h)
    r = _rep(dW, case["ref"]["dW"], case["ref"]["dW_c"])
    assert r["fail"] >= 0.9 * r["n"], r
