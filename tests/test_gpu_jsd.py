"""GPU parity of the generalized JSD against the fp64 oracle, through the C ABI.

Every element of JSD [N], ds and dt [N, V] is compared (bf16 and fp32) at interior
beta and at the two endpoint branches, on: a student/teacher pair with masked
columns and +1e4 rows, disjoint supports, identical rows (JSD 0, zero
gradients), a row spanning -3e38..3e38, undefined rows (NaN, all -inf), ragged
V, forced vocabulary splits, the element-wise (unaligned) path, 3-D [B, S, V]
views, a broadcast upstream gradient, a detached teacher, and the full
75968-column width.
"""

import numpy as np
import pytest
import torch

from oracle import compare, jsd as J
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu
NINF = float("-inf")


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _ok(rep, label):
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, (label, rep)
    print(label, {k: (rep[k] if not isinstance(rep[k], float) else round(rep[k], 4)) for k in rep}, flush=True)


def _pair(n, v, seed, dtype=torch.float32, special=True):
    gen = torch.Generator().manual_seed(seed)
    s = 3.0 * torch.randn(n, v, generator=gen)
    t = s + 1.0 * torch.randn(n, v, generator=gen)
    g = torch.randn(n, generator=gen)
    if special and n >= 8 and v >= 8:
        s[0] += 1e4
        t[0] += 1e4
        s[1, ::3] = NINF  # masked student columns
        t[2, 1::4] = NINF  # masked teacher columns
        s[3, : v // 2] = NINF  # disjoint supports
        t[3, v // 2:] = NINF
        t[4] = s[4]  # identical rows
        s[5] = -3e38
        s[5, 1] = 3e38
        t[5] = s[5]
        s[6, 2] = float("nan")  # undefined
        t[7] = NINF  # undefined (no live entry)
    return s.to(dtype), t.to(dtype), g


def _check(s_dev, t_dev, g_dev, s_host, t_host, g_host, beta, label, split=0, need_t=True, rows_chunk=64):
    kind = "bf16" if s_host.dtype == torch.bfloat16 else "f32"
    out, stats = B.jsd_fwd(s_dev, t_dev, beta, split)
    ds, dt = B.jsd_bwd(s_dev, t_dev, beta, stats, out, g_dev, need_t=need_t)
    torch.cuda.synchronize()
    hs = f64(s_host).reshape(-1, s_host.shape[-1])
    ht = f64(t_host).reshape(hs.shape)
    n = hs.shape[0]
    hg = np.full(n, float(g_host)) if g_host.numel() == 1 else g_host.double().reshape(n).numpy()
    go, gds = f64(out).reshape(n), f64(ds).reshape(hs.shape)
    gdt = f64(dt).reshape(hs.shape) if dt is not None else None
    for r0 in range(0, n, rows_chunk):
        sl = slice(r0, min(n, r0 + rows_chunk))
        o, _ = J.jsd_fwd(hs[sl], ht[sl], beta)
        _ok(compare.check(go[sl], o, J.cond_jsd_fwd(hs[sl], ht[sl], beta), "f32"), label + " jsd")
        rs, rt = J.jsd_bwd(hs[sl], ht[sl], hg[sl], beta)
        cs, ct = J.cond_jsd_bwd(hs[sl], ht[sl], hg[sl], beta)
        _ok(compare.check(gds[sl], rs, cs, kind), label + " ds")
        if gdt is not None:
            _ok(compare.check(gdt[sl], rt, ct, kind), label + " dt")
    assert need_t or dt is None


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("beta", [0.0, 0.3, 0.5, 0.9, 1.0])
def test_jsd_all_elements_special_rows(device, dtype, beta):
    print("jsd beta", beta, dtype, flush=True)
    s, t, g = _pair(64, 1024, seed=1, dtype=dtype)
    _check(s.to(device), t.to(device), g.to(device), s, t, g, beta, "pair64 beta=%g" % beta)


@pytest.mark.parametrize("v", [1, 7, 9, 100, 4097])
def test_jsd_ragged(device, v):
    s, t, g = _pair(9, v, seed=v, dtype=torch.bfloat16, special=v >= 8)
    _check(s.to(device), t.to(device), g.to(device), s, t, g, 0.4, "ragged v=%d" % v)


@pytest.mark.parametrize("split", [3, 16])
@pytest.mark.parametrize("offset", [0, 3])
def test_jsd_split_and_unaligned(device, split, offset):
    s, t, g = _pair(10, 5000, seed=7, dtype=torch.bfloat16)
    if offset:
        bs = torch.empty(s.numel() + offset, dtype=s.dtype, device=device)[offset:].view(s.shape)
        bt = torch.empty(t.numel() + offset, dtype=t.dtype, device=device)[offset:].view(t.shape)
        bs.copy_(s)
        bt.copy_(t)
    else:
        bs, bt = s.to(device), t.to(device)
    _check(bs, bt, g.to(device), s, t, g, 0.6, "split=%d off=%d" % (split, offset), split=split)


def test_jsd_3d_views_broadcast_g_detached_teacher(device):
    gen = torch.Generator().manual_seed(11)
    bs = 2.0 * torch.randn(3, 7, 900, generator=gen)
    bt = 2.0 * torch.randn(3, 7, 900, generator=gen)
    sv, tv = bs[:, :-1, :], bt[:, 1:, :]
    g = torch.tensor(1.5)
    ds_, dt_ = bs.to(device), bt.to(device)
    _check(ds_[:, :-1, :], dt_[:, 1:, :], g.to(device).expand(3, 6), sv, tv, g, 0.25, "3d views", need_t=False)


def test_jsd_near_endpoints(device):
    s, t, g = _pair(16, 3000, seed=12, dtype=torch.float32, special=False)
    for beta in (1e-3, 0.999):
        _check(s.to(device), t.to(device), g.to(device), s, t, g, beta, "beta=%g" % beta)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_jsd_full_width(device, dtype):
    """Every element of 48 rows 75968 wide (special rows included): whole batches and tiles,
    which on fp32 take the coalesced loads of the divergence pass and the backward."""
    s, t, g = _pair(48, 75968, seed=13, dtype=dtype)
    _check(s.to(device), t.to(device), g.to(device), s, t, g, 0.3, "full width %s" % dtype, rows_chunk=8)


def test_jsd_endpoint_branches_equal_kl_calls(device):
    s, t, g = _pair(32, 2000, seed=14, dtype=torch.bfloat16)
    sd, td, gd = s.to(device), t.to(device), g.to(device)
    j0, st0 = B.jsd_fwd(sd, td, 0.0)
    k0, sk0 = B.kl_fwd(td, sd)
    assert torch.equal(j0, k0) or torch.allclose(j0, k0, equal_nan=True, rtol=0, atol=0)
    j1, _ = B.jsd_fwd(sd, td, 1.0)
    k1, _ = B.kl_fwd(sd, td)
    assert torch.allclose(j1, k1, equal_nan=True, rtol=0, atol=0)
    ds, dt = B.jsd_bwd(sd, td, 0.0, st0, j0, gd)
    kt, ks = B.kl_bwd(td, sd, sk0, k0, gd)
    assert torch.equal(ds.view(torch.int16), ks.view(torch.int16)) and torch.equal(dt.view(torch.int16), kt.view(torch.int16))
