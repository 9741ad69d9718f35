"""The torch.autograd wrappers (vocab_wide_softmax_amd.ops) on the GPU.

Each op is differentiated through autograd and checked bit for bit against
the same forward and backward entry points called directly through the
binding: 3-D logits read in place as the causal-shift view ``x[:, :-1]`` (two
row strides; the gradient of the dropped position stays zero), gradients
asked for one input only, the expanded-scalar upstream gradient of a plain
``.sum()``, top-k ids dispatching to the multi-id op, and the fused
linear-logp. One op per family is also checked against the fp64 oracle
through autograd, so the wrappers cannot pass by agreeing with a wrong
binding call.
"""

import numpy as np
import pytest
import torch

from oracle import compare, reductions as R
from vocab_wide_softmax_amd import binding as B
from vocab_wide_softmax_amd import ops

pytestmark = pytest.mark.gpu


def _bits(x):
    return x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)


def _same(x, y):
    assert x.shape == y.shape and x.dtype == y.dtype, (x.shape, y.shape, x.dtype, y.dtype)
    assert torch.equal(_bits(x.contiguous()), _bits(y.contiguous()))


def _shifted(device, seed, b=3, s=41, v=1000, dtype=torch.bfloat16):
    gen = torch.Generator().manual_seed(seed)
    base = (2.5 * torch.randn(b, s + 1, v, generator=gen)).to(dtype).to(device)
    base2 = (base.float().cpu() + 0.7 * torch.randn(b, s + 1, v, generator=gen)).to(dtype).to(device)
    t = torch.randint(0, v, (b, s), generator=gen)
    t[0, 3] = -100
    w = torch.randn(b, s, generator=gen)
    return base, base2, t.to(device), w.to(device)


def _leaf(x):
    return x.detach().clone().requires_grad_(True)


def test_logprobs_shift_view(device):
    base, _, t, w = _shifted(device, 1)
    x = _leaf(base)
    view = x[:, :-1]
    out = ops.logprobs(view, t)
    (out * w).sum().backward()
    lp, st = B.logprobs_fwd(base[:, :-1], t)
    dz = B.logprobs_bwd(base[:, :-1], t, st, w)
    _same(out.detach(), lp)
    _same(x.grad[:, :-1], dz)
    assert torch.count_nonzero(x.grad[:, -1]) == 0
    # end to end against the oracle (the view's rows in order)
    z = base[:, :-1].float().cpu().double().reshape(-1, base.shape[-1]).numpy()
    tt, ww = t.cpu().reshape(-1).numpy(), w.cpu().double().reshape(-1).numpy()
    ref, _, _ = R.logprobs_fwd(z, tt, -100)
    rep = compare.check(out.detach().double().cpu().reshape(-1).numpy(), ref, R.cond_logprobs_fwd(z, tt, -100), "f32")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    gref = R.logprobs_bwd(z, tt, ww, -100)
    rep = compare.check(x.grad[:, :-1].double().cpu().reshape(-1, base.shape[-1]).numpy(), gref,
                        R.cond_logprobs_bwd(z, tt, ww, -100), "bf16")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep


def test_entropy_plain_sum_broadcast_gradient(device):
    base, _, _, _ = _shifted(device, 2)
    x = _leaf(base)
    H = ops.entropy(x)
    H.sum().backward()  # autograd hands the backward an expanded scalar
    Hd, st = B.entropy_fwd(base)
    dz = B.entropy_bwd(base, st, Hd, torch.ones(H.shape, device=device))
    _same(H.detach(), Hd)
    _same(x.grad, dz)


@pytest.mark.parametrize("need", ["both", "a", "b"])
def test_kl_partial_gradients(device, need):
    base, base2, _, w = _shifted(device, 3)
    a = _leaf(base) if need in ("both", "a") else base
    b = _leaf(base2) if need in ("both", "b") else base2
    out = ops.kl(a[:, :-1], b[:, :-1])
    (out * w).sum().backward()
    kl, st = B.kl_fwd(base[:, :-1], base2[:, :-1])
    da, db = B.kl_bwd(base[:, :-1], base2[:, :-1], st, kl, w)
    _same(out.detach(), kl)
    if need in ("both", "a"):
        _same(a.grad[:, :-1], da)
        assert torch.count_nonzero(a.grad[:, -1]) == 0
    if need in ("both", "b"):
        _same(b.grad[:, :-1], db)
    if need == "a":
        assert b.grad is None and not b.requires_grad
    if need == "b":
        assert a.grad is None and not a.requires_grad
    if need == "both":
        # end to end against the oracle
        za = base[:, :-1].float().cpu().double().reshape(-1, base.shape[-1]).numpy()
        zb = base2[:, :-1].float().cpu().double().reshape(-1, base.shape[-1]).numpy()
        ref = R.kl_fwd(za, zb)[0]
        rep = compare.check(out.detach().double().cpu().reshape(-1).numpy(), ref, R.cond_kl_fwd(za, zb), "f32")
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep


def test_jsd_student_only(device):
    base, base2, _, w = _shifted(device, 4, dtype=torch.float16)
    s = _leaf(base)
    out = ops.jsd(s, base2, beta=0.3)
    (out * w[:, :1].expand(-1, out.shape[1])).sum().backward()
    o, st = B.jsd_fwd(base, base2, 0.3)
    g = w[:, :1].expand(-1, out.shape[1]).contiguous()
    ds, dt = B.jsd_bwd(base, base2, 0.3, st, o, g, need_s=True, need_t=False)
    assert dt is None
    _same(out.detach(), o)
    _same(s.grad, ds)


def test_topk_dispatch(device):
    base, _, _, _ = _shifted(device, 5)
    gen = torch.Generator().manual_seed(6)
    ids = torch.randint(0, base.shape[-1], base.shape[:-1] + (4,), generator=gen)
    ids[1, 2, 1] = ids[1, 2, 0]  # a duplicate id: its gradients add
    ids[0, 0, :] = -100  # a fully ignored row
    ids = ids.to(device)
    wk = torch.randn(ids.shape, generator=gen).to(device)
    x = _leaf(base)
    out = ops.logprobs(x, ids)
    assert out.shape == ids.shape
    (out * wk).sum().backward()
    lp, st = B.logprobs_topk_fwd(base, ids)
    dz = B.logprobs_topk_bwd(base, ids, st, wk)
    _same(out.detach(), lp)
    _same(x.grad, dz)
    assert torch.count_nonzero(x.grad[0, 0]) == 0


def test_linear_logp_autograd(device):
    gen = torch.Generator().manual_seed(7)
    n, hid, v = 300, 192, 1100
    h0 = torch.randn(n, hid, generator=gen).bfloat16().to(device)
    W0 = (0.05 * torch.randn(v, hid, generator=gen)).bfloat16().to(device)
    t = torch.randint(0, v, (n,), generator=gen)
    t[5] = -100
    t, w = t.to(device), torch.randn(n, generator=gen).to(device)
    h, W = _leaf(h0), _leaf(W0)
    out = ops.linear_logp(h, W, t)
    (out * w).sum().backward()
    lp, st = B.linear_logp_fwd(h0, W0, t)
    dh, dW = B.linear_logp_bwd(h0, W0, t, st, w)
    _same(out.detach(), lp)
    _same(h.grad, dh)
    _same(W.grad, dW)
    # only W: no dh is formed
    W2 = _leaf(W0)
    (ops.linear_logp(h0, W2, t) * w).sum().backward()
    _same(W2.grad, dW)
    assert np.isfinite(out.detach().cpu().numpy()[t.cpu().numpy() != -100]).all()
