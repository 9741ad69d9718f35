"""50-digit brute-force reference with mpmath, used only to pin the fp64 oracle.

Written directly from the definitions (no max shift: mpmath has no exponent
range limit), so it shares no structure with the oracle's two-pass numpy
code. Gradients come from central differences at 50 digits, so they pin the
oracle's closed-form gradients without restating them.
"""

import math

import mpmath as mp

mp.mp.dps = 50
NEG_INF = float("-inf")


def _live(z):
    return [j for j, x in enumerate(z) if x != NEG_INF]


def logp_row(z):
    """log p_j = z_j - log sum_k e^{z_k}, -inf for masked entries."""
    zz = [mp.mpf(x) if x != NEG_INF else None for x in z]
    S = mp.fsum(mp.e ** x for x in zz if x is not None)
    lS = mp.log(S)
    return [(x - lS) if x is not None else mp.mpf("-inf") for x in zz]


def logprob(z, t):
    return logp_row(z)[t]


def entropy(z):
    lp = logp_row(z)
    return -mp.fsum(mp.e ** lp[j] * lp[j] for j in _live(z))


def kl(a, b):
    if any(a[j] != NEG_INF and b[j] == NEG_INF for j in range(len(a))):
        return mp.mpf("inf")
    la, lb = logp_row(a), logp_row(b)
    return mp.fsum(mp.e ** la[j] * (la[j] - lb[j]) for j in _live(a))


def grad(f, z, step=mp.mpf("1e-22")):
    """Central differences of f at z (masked entries keep gradient 0)."""
    out = []
    for j, x in enumerate(z):
        if x == NEG_INF:
            out.append(mp.mpf(0))
            continue
        zp = list(z)
        zm = list(z)
        zp[j] = mp.mpf(x) + step
        zm[j] = mp.mpf(x) - step
        out.append((f(zp) - f(zm)) / (2 * step))
    return out


def _mpify(z):
    return [mp.mpf(x) if x != NEG_INF else NEG_INF for x in z]


def logprob_grad(z, t):
    return grad(lambda zz: logprob(zz, t), _mpify(z))


def entropy_grad(z):
    return grad(entropy, _mpify(z))


def kl_grads(a, b):
    a, b = _mpify(a), _mpify(b)
    return grad(lambda aa: kl(aa, b), a), grad(lambda bb: kl(a, bb), b)


def to_float(v):
    return float(v) if not (mp.isinf(v) or mp.isnan(v)) else (math.inf if v > 0 else -math.inf)
