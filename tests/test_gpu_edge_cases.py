"""GPU edge cases and GPU-vs-GPU invariants, through the C ABI.

* ragged and tiny V, N = 1, the element-wise (unaligned) load path, forced splits, split
  parts whose columns are all -inf;
* rows the pages single out: a row spanning -3e38..3e38 (entropy 0, KL(p||p) 0,
  zero gradients), support mismatch with an underflowing p_A (+inf), all -inf
  rows, NaN / +inf entries, a target on a masked column, ignored and
  out-of-range targets, a broadcast upstream gradient;
* the empty batch (N = 0);
* bf16 inputs give bit-identical forward results to fp32 inputs holding the
  same values, and the bf16 gradient is the RNE of the fp32 one;
* repeated calls are bit-identical; KL(A||A) is exactly 0 with zero gradients.
"""

import numpy as np
import pytest
import torch

from parity import OPS, check_parity, f64, run_device, run_oracle
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu
NINF = float("-inf")


def _pair(n, v, seed, dtype=torch.float32):
    gen = torch.Generator().manual_seed(seed)
    a = 3.0 * torch.randn(n, v, generator=gen)
    b = a + 0.5 * torch.randn(n, v, generator=gen)
    t = torch.randint(0, v, (n,), generator=gen)
    g = torch.randn(n, generator=gen)
    return a.to(dtype), b.to(dtype), t, g


def _check_all_ops(a, b, t, g, device, split=0, kind=None, offset=0):
    """a, b host [n, v]; offset > 0 places the device rows at an element offset (unaligned path)."""
    kind = kind or ("bf16" if a.dtype == torch.bfloat16 else "f32")
    n, v = a.shape
    if offset:
        da_ = torch.empty(n * v + offset, dtype=a.dtype, device=device)[offset:].view(n, v)
        db_ = torch.empty(n * v + offset, dtype=a.dtype, device=device)[offset:].view(n, v)
        da_.copy_(a)
        db_.copy_(b)
    else:
        da_, db_ = a.to(device), b.to(device)
    dt = t.to(device)
    ha, hb = f64(a), f64(b)
    for op in OPS:
        dev = run_device(op, da_, db_, dt, g.to(device), split_hint=split)
        ora = run_oracle(op, ha, hb, t.numpy(), g.double().numpy())
        check_parity(dev, ora, kind, "%s n=%d v=%d split=%d off=%d" % (op, n, v, split, offset))


@pytest.mark.parametrize("v", [1, 7, 8, 9, 100, 1000, 4097])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_sizes(device, v, dtype):
    print("ragged v", v, dtype, flush=True)
    a, b, t, g = _pair(5, v, seed=v, dtype=dtype)
    _check_all_ops(a, b, t, g, device)


@pytest.mark.parametrize("split", [1, 3, 7])
@pytest.mark.parametrize("offset", [1, 3])
def test_unaligned_rows_and_splits(device, split, offset):
    print("unaligned offset", offset, "split", split, flush=True)
    a, b, t, g = _pair(6, 5000, seed=11, dtype=torch.bfloat16)
    _check_all_ops(a, b, t, g, device, split=split, offset=offset)


def test_single_row_long_vocab_split(device):
    a, b, t, g = _pair(1, 151936, seed=2, dtype=torch.bfloat16)
    assert B.split_parts(B.OP_KL, 1, 151936) > 1
    _check_all_ops(a, b, t, g, device)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fully_masked_split_parts(device, dtype):
    """Split parts whose columns are all -inf send the neutral partial (m = -inf, S = W = 0),
    which the merge must skip by the zero-weight rule: the first part masked in both inputs,
    the last part masked in both, and one part masked in A only (KL(B||A) = +inf there), with
    V = 1024 in 4 parts of 256 columns."""
    assert B.split_parts(B.OP_KL, 4, 1024, 4) == 4
    a, b, t, g = _pair(4, 1024, seed=31, dtype=torch.float32)
    a[0, :256] = NINF
    b[0, :256] = NINF
    t[0] = 300
    a[1, 768:] = NINF
    b[1, 768:] = NINF
    t[1] = 5
    a[2, 256:512] = NINF
    t[2] = 900
    _check_all_ops(a.to(dtype), b.to(dtype), t, g, device, split=4)


def _special_rows():
    v = 40
    a = torch.randn(8, v, generator=torch.Generator().manual_seed(1)) * 2
    b = a.clone() + 0.25
    a[0] = -3e38
    a[0, 5] = 3e38
    b[0] = a[0]
    b[1, 3] = NINF  # B masks a column A supports ...
    a[1, 3] = -1000.0  # ... whose p_A underflows
    a[2] = NINF
    b[2] = NINF  # all -inf row
    a[3, 7] = float("nan")
    a[4, 9] = float("inf")
    a[5, 11] = NINF  # target on a masked column (t set below)
    b[6] = NINF  # B fully masked: KL(A||B) = +inf
    a[7, :20] = NINF
    b[7, :20] = NINF  # masked in both
    t = torch.tensor([5, 0, 0, 0, 0, 11, -100, 200])  # 6: ignored, 7: out of range
    g = torch.tensor([1.0, -0.5, 2.0, 1.0, 1.0, 0.3, 1.0, 1.0])
    return a, b, t, g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("split", [1, 2])
def test_special_rows(device, dtype, split):
    print("special rows", dtype, split, flush=True)
    a, b, t, g = _special_rows()
    a, b = a.to(dtype), b.to(dtype)
    _check_all_ops(a, b, t, g, device, split=split)
    # the pages' exact values on the extreme-range row
    H, st = B.entropy_fwd(a.to(device))
    assert H[0].item() == 0.0
    kl, st = B.kl_fwd(a.to(device)[:1], a.to(device)[:1])
    assert kl[0].item() == 0.0
    dz = B.entropy_bwd(a.to(device)[:1], B.entropy_fwd(a.to(device)[:1])[1], H[:1], g[:1].to(device))
    assert torch.all(dz == 0)
    klab, _ = B.kl_fwd(a.to(device), b.to(device))
    assert klab[1].item() == float("inf") and klab[6].item() == float("inf")


def test_broadcast_upstream_gradient(device):
    a, b, t, g = _pair(4, 333, seed=3)
    da = a.to(device)
    H, st = B.entropy_fwd(da)
    g1 = torch.tensor(0.75, device=device).expand(4)
    d1 = B.entropy_bwd(da, st, H, g1)
    d2 = B.entropy_bwd(da, st, H, torch.full((4,), 0.75, device=device))
    assert torch.equal(d1, d2)


def test_empty_batch(device):
    z = torch.empty(0, 100, device=device)
    H, st = B.entropy_fwd(z)
    assert H.numel() == 0
    dz = B.entropy_bwd(z, st, H, torch.empty(0, device=device))
    assert dz.shape == (0, 100)
    kl, st = B.kl_fwd(z, z)
    da, db = B.kl_bwd(z, z, st, kl, torch.empty(0, device=device))
    assert da.shape == (0, 100)


def test_dtype_invariance_and_rne(device):
    """bf16 input vs the same values in fp32: forward bit-identical, bf16 grad = RNE(fp32 grad)."""
    a, b, t, g = _pair(64, 75968, seed=7, dtype=torch.bfloat16)
    a32, b32 = a.float(), b.float()
    for op in OPS:
        r16 = run_device(op, a.to(device), b.to(device), t.to(device), g.to(device))
        r32 = run_device(op, a32.to(device), b32.to(device), t.to(device), g.to(device))
        assert np.array_equal(r16["out"], r32["out"], equal_nan=True), op
        assert np.array_equal(r16["stats"], r32["stats"], equal_nan=True), op
        for x16, x32 in zip(r16["grads"], r32["grads"]):
            rne = torch.from_numpy(x32).float().to(torch.bfloat16).double().numpy()
            assert np.array_equal(x16, rne, equal_nan=True), op


def test_repeatable_and_kl_self_zero(device):
    a, b, t, g = _pair(300, 20000, seed=9, dtype=torch.bfloat16)
    da, db, dt, dg = a.to(device), b.to(device), t.to(device), g.to(device)
    for op in OPS:
        r1 = run_device(op, da, db, dt, dg)
        r2 = run_device(op, da, db, dt, dg)
        assert np.array_equal(r1["out"], r2["out"], equal_nan=True)
        for x, y in zip(r1["grads"], r2["grads"]):
            assert np.array_equal(x, y, equal_nan=True)
    kl, st = B.kl_fwd(da, da)
    assert torch.all(kl == 0)
    ga, gb = B.kl_bwd(da, da, st, kl, dg)
    assert torch.all(ga == 0) and torch.all(gb == 0)


def test_split_matches_unsplit(device):
    a, b, t, g = _pair(16, 75968, seed=4, dtype=torch.bfloat16)
    da, db = a.to(device), b.to(device)
    H1, s1 = B.entropy_fwd(da, split_hint=1)
    H8, s8 = B.entropy_fwd(da, split_hint=8)
    assert torch.equal(s1[:, 0], s8[:, 0])
    torch.testing.assert_close(H1, H8, rtol=2e-6, atol=0)
    k1, _ = B.kl_fwd(da, db, split_hint=1)
    k8, _ = B.kl_fwd(da, db, split_hint=8)
    torch.testing.assert_close(k1, k8, rtol=1e-4, atol=1e-6)


def _gap_rows(n, v, seed, lo=86.0, hi=104.0):
    """Rows with one maximum at 0 and the rest spread over log-probability gaps of lo..hi nats,
    so that p lies in [e^-104, e^-86]: below the smallest normal fp32 (2^-126 = e^-87.3) for most
    columns, where the gradient is a subnormal that bf16 still holds (down to 2^-133 = e^-92.2)."""
    gen = torch.Generator().manual_seed(seed)
    a = -(lo + (hi - lo) * torch.rand(n, v, generator=gen))
    a[:, 0] = 0.0
    b = a + 0.5 * torch.randn(n, v, generator=gen)
    b[:, 0] = 0.0
    t = torch.randint(1, v, (n,), generator=gen)
    g = torch.randn(n, generator=gen) * 1000.0  # large enough that g p is a normal number on some columns
    return a, b, t, g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_subnormal_probabilities_in_gradients(device, dtype):
    """Gradients built on probabilities between 2^-149 and 2^-126: the hardware exponential flushes
    results there to 0, so the backward passes rescale such arguments; every gradient element
    (logprobs, entropy, both KL directions) must still pass the rule, including the bf16
    subnormals and the normal-range products g p (log p - ...)."""
    a, b, t, g = _gap_rows(6, 1500, seed=41)
    a, b = a.to(dtype), b.to(dtype)
    print("subnormal p", dtype, flush=True)
    _check_all_ops(a, b, t, g, device)
    # the top-k backward and the JSD backward recompute p the same way
    from oracle import compare, jsd as J, topk as TK

    ids = torch.stack([t, (t + 7) % 1500, t], dim=1)
    gk = torch.randn(6, 3, generator=torch.Generator().manual_seed(3)) * 1000.0
    da_, db_ = a.to(device), b.to(device)
    lp, st = B.logprobs_topk_fwd(da_, ids.to(device), -100)
    dz = B.logprobs_topk_bwd(da_, ids.to(device), st, gk.to(device), -100)
    ha, hb, hi, hg = f64(a), f64(b), ids.numpy(), gk.double().numpy()
    kind = "bf16" if dtype == torch.bfloat16 else "f32"
    rep = compare.check(f64(dz), TK.logprobs_topk_bwd(ha, hi, hg), TK.cond_logprobs_topk_bwd(ha, hi, hg), kind)
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    out, st = B.jsd_fwd(da_, db_, 0.4)
    ds, dt = B.jsd_bwd(da_, db_, 0.4, st, out, g.to(device))
    rs, rt = J.jsd_bwd(ha, hb, g.double().numpy(), 0.4)
    cs, ct = J.cond_jsd_bwd(ha, hb, g.double().numpy(), 0.4)
    for x, y, c in ((ds, rs, cs), (dt, rt, ct)):
        rep = compare.check(f64(x), y, c, kind)
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    if dtype == torch.bfloat16:
        # the case is not vacuous: the oracle's entropy gradient has normal-range entries below
        # e^-87.3 probability, which a flushed exponential would zero
        from oracle import reductions as R

        ge = R.entropy_bwd(ha, g.double().numpy())
        p = np.exp(ha - np.log(np.exp(ha).sum(axis=1, keepdims=True)))
        assert np.count_nonzero((p < 2.0 ** -126) & (compare.bf16_rne(ge) != 0)) > 1000
