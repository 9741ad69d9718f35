"""fp16 inputs and batch invariance, through the C ABI.

fp16 (the JSD pull request on PR #8838 validates FP32/FP16/BF16 kernels):
every op's outputs and fp16 gradients against the fp64 oracle (gradients
rounded to nearest even in fp16), ragged V, special rows scaled to the fp16
range, and the fp16 -> fp32 dtype invariance of the forward, for both
forward workgroup widths (the 512-lane one of large automatic batches is also
held to the oracle on every element).

Batch invariance (the remark on PR #8838 about checking batch invariance for
RL rollouts): with split_hint = SPLIT_INVARIANT the vocabulary is cut into
segments that depend on V alone, so a row's outputs are bitwise identical
whether it is computed in a batch of 512 rows, of 37 rows, or alone; the
backward passes are per element and follow. Checked for logprobs (single and
top-k), entropy, KL and JSD.
"""

import numpy as np
import pytest
import torch

from oracle import compare, jsd as J, topk as TK
from parity import OPS, check_parity, f64, run_device, run_oracle
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu
NINF = float("-inf")
INV = B.SPLIT_INVARIANT


def _pair(n, v, seed, scale=3.0):
    gen = torch.Generator().manual_seed(seed)
    a = scale * torch.randn(n, v, generator=gen)
    b = a + 0.5 * torch.randn(n, v, generator=gen)
    t = torch.randint(0, v, (n,), generator=gen)
    g = torch.randn(n, generator=gen)
    return a, b, t, g


def _all_ops(a, b, t, g, device, split=0):
    for op in OPS:
        dev = run_device(op, a.to(device), b.to(device), t.to(device), g.to(device), split_hint=split)
        ora = run_oracle(op, f64(a), f64(b), t.numpy(), g.double().numpy())
        check_parity(dev, ora, "f16", "%s fp16 v=%d split=%d" % (op, a.shape[1], split))


@pytest.mark.parametrize("v", [7, 100, 4097, 75968])
def test_fp16_all_ops(device, v):
    n = 24 if v == 75968 else 12
    a, b, t, g = _pair(n, v, seed=v)
    a[0] += 2000.0  # a large common offset (fp16 spacing is 1 there)
    b[0] += 2000.0
    if v >= 100:
        b[1, :: v // 10] = NINF
        a[2, 3] = NINF
        t[2] = 3  # target on a masked column
        t[3] = -100
    _all_ops(a.half(), b.half(), t, g, device)


@pytest.mark.parametrize("split", [1, 5, INV])
def test_fp16_special_rows_and_splits(device, split):
    v = 40
    a, b, t, g = _pair(6, v, seed=2, scale=2.0)
    a[0] = -65504.0  # a row spanning the whole fp16 range: one-hot
    a[0, 5] = 65504.0
    b[0] = a[0]
    a[1] = NINF
    b[1] = NINF
    a[2, 4] = float("nan")
    b[3] = NINF  # B fully masked: KL(A||B) = +inf
    t[4] = 200  # out of range
    _all_ops(a.half(), b.half(), t, g, device, split=split)


def test_fp16_forward_matches_fp32_bitwise(device):
    """The element -> lane map does not depend on the dtype: fp16 inputs and the same values
    in fp32 give identical forward results, and the fp16 gradient is the RNE of the fp32 one.
    At this width the fp32 forward loads its whole batches coalesced and regroups them across
    lanes, so special values sit inside those batches too."""
    a, b, t, g = _pair(32, 75968, seed=5, scale=2.0)
    a[0, 3000:3100] = NINF  # masked columns inside a whole batch
    b[0, 3050:3200] = NINF  # some live A columns masked in B: KL = +inf
    a[1, 9000] = float("nan")
    b[2] = NINF  # B fully masked
    a[3] = -60000.0  # one-hot row
    a[3, 20001] = 60000.0
    b[3] = a[3]
    a[4] += 3e4  # large common offset
    b[4] += 3e4
    a[5, ::2] = NINF  # every other column masked
    a16, b16 = a.half(), b.half()
    for op in OPS:
        r16 = run_device(op, a16.to(device), b16.to(device), t.to(device), g.to(device))
        r32 = run_device(op, a16.float().to(device), b16.float().to(device), t.to(device), g.to(device))
        assert np.array_equal(r16["out"], r32["out"], equal_nan=True), op
        for x16, x32 in zip(r16["grads"], r32["grads"]):
            rne = torch.from_numpy(x32).float().half().double().numpy()
            assert np.array_equal(x16, rne, equal_nan=True), op


@pytest.mark.parametrize("v", [4104, 4099])
def test_wide_forward_dtype_identity(device, v):
    """From 2048 rows up the automatic forward runs 512-lane workgroups (another element -> lane
    map than the 256-lane one the smaller batches above take): bf16 and fp16 inputs still give
    the forward of the same values in fp32 bit for bit, and their gradients are the RNE of the
    fp32 ones, on whole vector batches (v = 4104) and on the predicated path of rows whose
    pitch is not a whole number of 16-byte groups (v = 4099)."""
    a, b, t, g = _pair(2048, v, seed=9, scale=2.0)
    a[0, 100:300] = NINF
    b[1, 50:90] = NINF
    a[2] += 3e3
    b[2] += 3e3
    a[3, ::3] = NINF
    for lo in (torch.bfloat16, torch.float16):
        al, bl = a.to(lo), b.to(lo)
        print("wide forward identity", v, lo, flush=True)
        for op in OPS:
            rl = run_device(op, al.to(device), bl.to(device), t.to(device), g.to(device))
            r32 = run_device(op, al.float().to(device), bl.float().to(device), t.to(device), g.to(device))
            assert np.array_equal(rl["out"], r32["out"], equal_nan=True), (op, lo)
            assert np.array_equal(rl["stats"], r32["stats"], equal_nan=True), (op, lo)
            for xl, x32 in zip(rl["grads"], r32["grads"]):
                rne = torch.from_numpy(x32).float().to(lo).double().numpy()
                assert np.array_equal(xl, rne, equal_nan=True), (op, lo)


def test_wide_forward_parity(device):
    """The 512-lane forward (2048 rows, automatic split) against the fp64 oracle on every row
    and element, fp32 logits with a ragged vocabulary (the predicated path) and special rows."""
    a, b, t, g = _pair(2048, 4099, seed=10, scale=3.0)
    a[0, 7:4000:5] = NINF
    b[5] = NINF
    t[6] = -100
    a[7] += 1e4
    b[7] += 1e4
    for op in OPS:
        dev = run_device(op, a.to(device), b.to(device), t.to(device), g.to(device))
        ora = run_oracle(op, f64(a), f64(b), t.numpy(), g.double().numpy())
        check_parity(dev, ora, "f32", "%s wide fp32 2048x4099" % op)


def test_fp16_topk_and_jsd(device):
    gen = torch.Generator().manual_seed(6)
    s = (2.0 * torch.randn(20, 3000, generator=gen)).half()
    t = (s.float() + torch.randn(20, 3000, generator=gen)).half()
    ids = torch.randint(0, 3000, (20, 6), generator=gen)
    ids[0, 1] = ids[0, 2]
    ids[1, :] = -100
    gk = torch.randn(20, 6, generator=gen)
    logp, st = B.logprobs_topk_fwd(s.to(device), ids.to(device), -100)
    dz = B.logprobs_topk_bwd(s.to(device), ids.to(device), st, gk.to(device), -100)
    hs, hi, hg = f64(s), ids.numpy(), gk.double().numpy()
    rep = compare.check(f64(logp), TK.logprobs_topk_fwd(hs, hi)[0], TK.cond_logprobs_topk_fwd(hs, hi), "f32")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    rep = compare.check(f64(dz), TK.logprobs_topk_bwd(hs, hi, hg), TK.cond_logprobs_topk_bwd(hs, hi, hg), "f16")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    g = torch.randn(20, generator=gen)
    out, st = B.jsd_fwd(s.to(device), t.to(device), 0.4)
    ds, dt = B.jsd_bwd(s.to(device), t.to(device), 0.4, st, out, g.to(device))
    ht, hgj = f64(t), g.double().numpy()
    rep = compare.check(f64(out), J.jsd_fwd(hs, ht, 0.4)[0], J.cond_jsd_fwd(hs, ht, 0.4), "f32")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    rs, rt = J.jsd_bwd(hs, ht, hgj, 0.4)
    cs, ct = J.cond_jsd_bwd(hs, ht, hgj, 0.4)
    for x, y, c in ((ds, rs, cs), (dt, rt, ct)):
        rep = compare.check(f64(x), y, c, "f16")
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep


def _bits(x):
    return x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)


def _rows_of(x, idx):
    return x[idx].contiguous()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_batch_invariance(device, dtype):
    """A row's results do not depend on the batch around it in the invariant split mode."""
    n, v = 512, 75968
    a, b, t, g = _pair(n, v, seed=8)
    a[3] += 1e4
    b[3] += 1e4
    a, b = a.to(dtype), b.to(dtype)
    sub = torch.tensor([3, 17, 100, 101, 255, 256, 300, 511] + list(range(400, 429)))  # 37 rows
    one = torch.tensor([101])
    ids = torch.randint(0, v, (n, 4), generator=torch.Generator().manual_seed(9))
    da, db, dt, dg, di = a.to(device), b.to(device), t.to(device), g.to(device), ids.to(device)

    def everything(x, y, tt, gg, ii):
        res = {}
        res["logprobs"] = B.logprobs_fwd(x, tt, -100, INV)[0]
        res["topk"] = B.logprobs_topk_fwd(x, ii, -100, INV)[0]
        H, st = B.entropy_fwd(x, INV)
        res["entropy"] = H
        res["entropy_stats"] = st
        kl, stk = B.kl_fwd(x, y, INV)
        res["kl"] = kl
        res["kl_stats"] = stk
        res["kl_da"], res["kl_db"] = B.kl_bwd(x, y, stk, kl, gg)
        jo, sj = B.jsd_fwd(x, y, 0.3, INV)
        res["jsd"] = jo
        res["jsd_stats"] = sj
        res["jsd_ds"], res["jsd_dt"] = B.jsd_bwd(x, y, 0.3, sj, jo, gg)
        return res

    full = everything(da, db, dt, dg, di)
    for idx in (sub, one):
        idd = idx.to(device)
        part = everything(_rows_of(da, idd), _rows_of(db, idd), _rows_of(dt, idd), _rows_of(dg, idd),
                          _rows_of(di, idd))
        for k, val in part.items():
            assert torch.equal(_bits(val), _bits(full[k][idd])), (k, len(idx))
    assert B.split_parts(B.OP_KL, 512, v, INV) == B.split_parts(B.OP_KL, 1, v, INV) == 3
