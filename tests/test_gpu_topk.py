"""GPU parity of the multi-id (top-k) logprobs against the fp64 oracle, through the C ABI.

Cases (the pages' test list includes repeated ids, ignored ids and rows with every
id ignored): duplicates, ignored slots, a fully ignored row, an out-of-range
slot (NaN logp, NaN gradient row), a target on a masked column, a +1e4 row,
ragged V, the element-wise (unaligned) load path, forced vocabulary splits, a
3-D [B, S, V] view with strided ids, a broadcast upstream gradient, the largest
K of each backward kernel (64 and 2048) with every id in one column tile,
K = 64 and 65 on either side of the kernel switch, and the full 75968-column width.
Every element of logp [N, K] and dz [N, V] is compared.
"""

import numpy as np
import pytest
import torch

from oracle import compare, topk as TK
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu
IGN = -100


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _ok(rep, label):
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, (label, rep)
    print(label, {k: (rep[k] if not isinstance(rep[k], float) else round(rep[k], 4)) for k in rep}, flush=True)


def _case(n, v, K, seed, dtype):
    gen = torch.Generator().manual_seed(seed)
    z = 3.0 * torch.randn(n, v, generator=gen)
    ids = torch.randint(0, v, (n, K), generator=gen)
    g = torch.randn(n, K, generator=gen)
    if n > 4 and K > 3:
        ids[0, 1] = ids[0, 3]  # duplicate
        ids[1, :] = ids[1, 0]  # every slot the same id
        ids[2, 2] = IGN
        ids[3, :] = IGN  # fully ignored row
        z[4] += 1e4
    if n > 6:
        ids[5, K - 1] = v  # out of range: NaN slot, NaN gradient row
        z[6, :: max(1, v // 7)] = float("-inf")
        ids[6, 0] = 0  # target on a masked column
    return z.to(dtype), ids, g


def _run_and_check(z_dev, ids_dev, g_dev, z_host, ids_host, g_host, label, split=0):
    kind = "bf16" if z_host.dtype == torch.bfloat16 else "f32"
    logp, stats = B.logprobs_topk_fwd(z_dev, ids_dev, IGN, split)
    dz = B.logprobs_topk_bwd(z_dev, ids_dev, stats, g_dev, IGN)
    torch.cuda.synchronize()
    hz = f64(z_host).reshape(-1, z_host.shape[-1])
    hi = ids_host.reshape(hz.shape[0], -1).numpy()
    if g_host.numel() == 1:
        hg = np.full(hi.shape, float(g_host.reshape(-1)[0]))
    else:
        hg = g_host.double().reshape(hi.shape).numpy()
    out, m, ls = TK.logprobs_topk_fwd(hz, hi, IGN)
    _ok(compare.check(f64(logp).reshape(hi.shape), out, TK.cond_logprobs_topk_fwd(hz, hi, IGN), "f32"),
        label + " logp")
    _ok(compare.check(f64(dz).reshape(hz.shape), TK.logprobs_topk_bwd(hz, hi, hg, IGN),
                      TK.cond_logprobs_topk_bwd(hz, hi, hg, IGN), kind), label + " dz")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("v,K", [(1024, 8), (4097, 5), (9, 3), (75968, 16), (9000, 64), (9000, 65)])
def test_topk_all_elements(device, dtype, v, K):
    n = 24 if v == 75968 else 40
    print("topk v", v, "K", K, dtype, flush=True)
    z, ids, g = _case(n, v, K, seed=v + K, dtype=dtype)
    _run_and_check(z.to(device), ids.to(device), g.to(device), z, ids, g, "v=%d K=%d" % (v, K))


@pytest.mark.parametrize("n", [40, 2048])
@pytest.mark.parametrize("K", [256, 257])
def test_topk_slot_limit_of_the_fused_forward(device, K, n):
    """Unsplit rows: K = 256 slots are written by the forward pass itself (one per lane), K = 257
    by the statistics pass and the gather launch; every element against the oracle. 40 rows run
    the 256-lane forward, 2048 rows the 512-lane one (its first 256 lanes hold the slots)."""
    z, ids, g = _case(n, 1024, K, seed=K + n, dtype=torch.bfloat16)
    assert B.split_parts(B.OP_LOGPROBS, n, 1024) == 1
    _run_and_check(z.to(device), ids.to(device), g.to(device), z, ids, g, "K=%d n=%d" % (K, n))


@pytest.mark.parametrize("split", [3, 16])
def test_topk_forced_split(device, split):
    z, ids, g = _case(12, 5000, 6, seed=5, dtype=torch.bfloat16)
    _run_and_check(z.to(device), ids.to(device), g.to(device), z, ids, g, "split=%d" % split, split=split)


def test_topk_unaligned_rows(device):
    z, ids, g = _case(10, 3001, 4, seed=6, dtype=torch.bfloat16)
    buf = torch.empty(z.numel() + 3, dtype=z.dtype, device=device)
    zd = buf[3:].view(z.shape)
    zd.copy_(z)
    _run_and_check(zd, ids.to(device), g.to(device), z, ids, g, "unaligned")


def test_topk_3d_view_and_strided_ids(device):
    gen = torch.Generator().manual_seed(9)
    base = 3.0 * torch.randn(2, 9, 700, generator=gen)
    ids_base = torch.randint(0, 700, (2, 9, 12), generator=gen)
    ids_base[0, 2, ::2] = IGN
    g = torch.randn(2, 8, 4, generator=gen)
    zb, ib = base.to(device), ids_base.to(device)
    zv, iv = zb[:, :-1, :], ib[:, 1:, ::3]  # two row strides; ids with row and slot strides
    assert iv.stride(2) == 3
    _run_and_check(zv, iv, g.to(device), base[:, :-1, :], ids_base[:, 1:, ::3], g, "3d view")


def test_topk_broadcast_upstream_gradient(device):
    z, ids, _ = _case(16, 2000, 5, seed=7, dtype=torch.float32)
    g = torch.tensor(0.75)
    gd = g.to(device).expand(16, 5)
    _run_and_check(z.to(device), ids.to(device), gd, z, ids, g, "broadcast g")


@pytest.mark.parametrize("K", [64, 2048])
def test_topk_max_k_all_in_one_tile(device, K):
    """The largest K of each backward kernel (slots in lane registers up to 64, in LDS above)
    with every id in one column tile and many duplicates."""
    n, v = 3, 6000
    gen = torch.Generator().manual_seed(8)
    z = 2.0 * torch.randn(n, v, generator=gen)
    ids = torch.randint(4096, 4200, (n, K), generator=gen)  # all in one column tile, many duplicates
    ids[1, ::5] = IGN
    g = torch.randn(n, K, generator=gen)
    _run_and_check(z.to(device), ids.to(device), g.to(device), z, ids, g, "K=%d one tile" % K)


def test_topk_single_slot_matches_single_id_op(device):
    z, ids, g = _case(32, 3000, 1, seed=10, dtype=torch.bfloat16)
    zd, td, gd = z.to(device), ids[:, 0].contiguous().to(device), g[:, 0].contiguous().to(device)
    lp1, st1 = B.logprobs_fwd(zd, td, IGN)
    lpk, stk = B.logprobs_topk_fwd(zd, ids.to(device), IGN)
    assert torch.equal(st1, stk)
    d1 = B.logprobs_bwd(zd, td, st1, gd, IGN)
    dk = B.logprobs_topk_bwd(zd, ids.to(device), stk, g.to(device), IGN)
    # same statistics; the one-hot term is formed as fma(-g, p, g) here and g (1 - p) there
    rep = compare.check(f64(dk), f64(d1).astype(np.float64), np.abs(f64(d1)) + 1e-30, "bf16")
    assert rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0 and rep["fail"] == 0, rep
    assert torch.allclose(lpk[:, 0], lp1, rtol=2e-6, atol=2e-6, equal_nan=True)


@pytest.mark.parametrize("split", [0, 4])
def test_ignore_index_inside_the_vocabulary(device, split):
    """ignore_index may name a real column: slots (and single targets) equal to it give 0 and no
    gradient, other slots on that column's neighbours are ordinary. Unsplit rows take the forward's
    own slot outputs, split rows the statistics pass and the gather launch."""
    import oracle.reductions as R

    ign = 7
    n, v = 24, 9000
    gen = torch.Generator().manual_seed(21)
    z = 2.0 * torch.randn(n, v, generator=gen)
    ids = torch.randint(0, v, (n, 5), generator=gen)
    ids[0, 1] = ign
    ids[1, :] = ign  # fully ignored row
    ids[2, 3] = ign - 1
    ids[3, 0] = ign + 1
    g = torch.randn(n, 5, generator=gen)
    zd, idd, gd = z.to(device), ids.to(device), g.to(device)
    logp, stats = B.logprobs_topk_fwd(zd, idd, ign, split)
    dz = B.logprobs_topk_bwd(zd, idd, stats, gd, ign)
    torch.cuda.synchronize()
    hz, hi, hg = f64(z), ids.numpy(), g.double().numpy()
    out, _, _ = TK.logprobs_topk_fwd(hz, hi, ign)
    _ok(compare.check(f64(logp), out, TK.cond_logprobs_topk_fwd(hz, hi, ign), "f32"), "top-k ign=7")
    _ok(compare.check(f64(dz), TK.logprobs_topk_bwd(hz, hi, hg, ign), TK.cond_logprobs_topk_bwd(hz, hi, hg, ign),
                      "f32"), "top-k ign=7 dz")
    assert float(logp[0, 1]) == 0.0 and bool((logp[1] == 0).all())
    # single target per row
    t = ids[:, 0].contiguous()
    lp1, st1 = B.logprobs_fwd(zd, t.to(device), ign, split)
    d1 = B.logprobs_bwd(zd, t.to(device), st1, gd[:, 0].contiguous(), ign)
    torch.cuda.synchronize()
    o1, _, _ = R.logprobs_fwd(hz, t.numpy(), ignore_index=ign)
    _ok(compare.check(f64(lp1), o1, R.cond_logprobs_fwd(hz, t.numpy(), ignore_index=ign), "f32"), "single ign=7")
    assert float(lp1[1]) == 0.0 and bool((d1[1] == 0).all())
