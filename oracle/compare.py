"""Element-wise acceptance rule for parity tests (test infrastructure only).

Tolerances (stated for this path; the pages report errors, not a rule):
* fp32 outputs x against the float64 value y pass when
    |x - y| <= 2e-5 |y| + 2^-126                         (strict), or
    |x - y| <= 2e-5 |y| + 64 eps32 c                     (conditioned),
  where c is the conditioning scale of the element (sum of magnitudes of the
  terms its formula combines) and eps32 = 2^-23.
* bf16 outputs pass when
    |x - rne(y)| <= ulp_bf16(rne(y))                     (strict), or
    |x - y| <= ulp_bf16(rne(y)) + 64 eps32 c             (conditioned),
  with rne(y) the bf16 value nearest to y, ties to even (a bf16 gradient is its
  fp32 value rounded that way, as the review comment of PR #8838 observes).
* fp16 outputs pass by the bf16 rule with fp16 rounding and spacing
    (|x - rne16(y)| <= ulp_f16(rne16(y)), or the conditioned form).
* NaN positions must match exactly, and so must +inf / -inf positions.

The conditioned branch exists because a purely relative bound cannot be met
where the exact value is a near-cancelling difference (e.g. g (p_B - p_A)
with B close to A, or an entropy gradient whose exact value is 0).
"""

import numpy as np

EPS32 = 2.0 ** -23
REL32 = 2e-5
COND = 64.0 * EPS32

__all__ = ["EPS32", "bf16_rne", "ulp_bf16", "f16_rne", "ulp_f16", "check", "bf16_bits_to_f64", "f64_to_bf16_bits"]


def bf16_rne(y):
    """Round float64 values to the nearest bf16 value, ties to even (exact, no double rounding)."""
    y = np.asarray(y, dtype=np.float64)
    out = np.array(y, dtype=np.float64, copy=True)
    fin = np.isfinite(y) & (y != 0)
    a = np.abs(y[fin])
    e = np.floor(np.log2(a))
    # guard floor(log2) at exact powers of two / rounding of log2
    e = np.where(2.0 ** e > a, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= a, e + 1, e)
    e = np.maximum(e, -126.0)
    ulp = 2.0 ** (e - 7)
    r = np.rint(a / ulp) * ulp  # a/ulp is exact (power-of-two scaling); rint is ties-to-even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[fin] = np.sign(y[fin]) * r
    return out


def ulp_bf16(v):
    """Spacing of bf16 values at |v| (v a bf16 value or 0)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.where(v > 0, e, -126.0)
    e = np.maximum(e, -126.0)
    return 2.0 ** (e - 7)


def f16_rne(y):
    """Round float64 values to the nearest IEEE half value, ties to even; beyond the largest
    half (65504) values that round up to 2^16 become inf."""
    y = np.asarray(y, dtype=np.float64)
    out = np.array(y, dtype=np.float64, copy=True)
    fin = np.isfinite(y) & (y != 0)
    a = np.abs(y[fin])
    e = np.floor(np.log2(a))
    e = np.where(2.0 ** e > a, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= a, e + 1, e)
    e = np.maximum(e, -14.0)  # subnormal halves share the spacing 2^-24
    ulp = 2.0 ** (e - 10)
    r = np.rint(a / ulp) * ulp
    r = np.where(r > 65504.0, np.inf, r)
    out[fin] = np.sign(y[fin]) * r
    return out


def ulp_f16(v):
    """Spacing of half values at |v| (v a half value or 0)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.where(v > 0, e, -14.0)
    e = np.maximum(e, -14.0)
    return 2.0 ** (e - 10)


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 values -> uint16 bf16 patterns, rounding to nearest even."""
    r = bf16_rne(x).astype(np.float32)  # exact: bf16 values are fp32 values
    bits = (r.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float64))
    bits[nan] = 0x7FC0
    return bits


def check(x, y, c, kind):
    """Compare device values x with oracle values y under the rule above.

    kind is "f32", "bf16" or "f16". Returns a dict with the element count, the
    number of elements missing the strict bound, the number failing both bounds,
    the NaN / inf placement mismatches, and the worst ratio of error to allowance.
    For fp32 values it also reports max_rel, the largest |x - y| / |y| over finite
    nonzero y: the form of the fp32 output errors against a float64 CPU reference
    that the description of PR #8838 quotes under "Numerics" (None for bf16 and fp16,
    whose relative error is the output rounding itself).
    """
    cfac = COND
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    c = np.asarray(c, dtype=np.float64).ravel()
    if c.size == 1 and x.size != 1:
        c = np.full(x.shape, float(c[0]))
    assert x.shape == y.shape == c.shape, (x.shape, y.shape, c.shape)
    nan_mis = int(np.count_nonzero(np.isnan(x) != np.isnan(y)))
    inf_mis = int(np.count_nonzero((np.isposinf(x) != np.isposinf(y)) | (np.isneginf(x) != np.isneginf(y))))
    fin = np.isfinite(x) & np.isfinite(y)
    xf, yf = x[fin], y[fin]
    cf = np.where(np.isfinite(c[fin]), c[fin], 0.0)
    if kind == "f32":
        err = np.abs(xf - yf)
        strict = REL32 * np.abs(yf) + 2.0 ** -126
        cond = REL32 * np.abs(yf) + cfac * cf
        strict_ok = err <= strict
        ok = strict_ok | (err <= cond)
        allow = np.maximum(strict, cond)
    elif kind in ("bf16", "f16"):
        r = bf16_rne(yf) if kind == "bf16" else f16_rne(yf)
        u = ulp_bf16(r) if kind == "bf16" else ulp_f16(np.where(np.isfinite(r), r, 65504.0))
        strict_ok = np.abs(xf - r) <= u
        cond = u + cfac * cf
        ok = strict_ok | (np.abs(xf - yf) <= cond)
        err = np.minimum(np.abs(xf - r), np.abs(xf - yf))
        allow = cond
    else:
        raise ValueError(kind)
    worst = float(np.max(err / allow)) if err.size else 0.0
    max_rel = None
    if kind == "f32":
        nz = yf != 0
        max_rel = float(np.max(np.abs(xf[nz] - yf[nz]) / np.abs(yf[nz]))) if np.any(nz) else 0.0
    return {
        "n": int(x.size),
        "strict_miss": int(np.count_nonzero(~strict_ok)),
        "fail": int(np.count_nonzero(~ok)),
        "nan_mismatch": nan_mis,
        "inf_mismatch": inf_mis,
        "worst": worst,
        "max_rel": max_rel,
    }
