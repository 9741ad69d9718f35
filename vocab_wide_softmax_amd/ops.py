"""torch.autograd wrappers over the libvws entry points.

``logprobs(z, t)``, ``entropy(z)`` and ``kl(a, b)`` return fp32 per-token
values (shape of the logits without the last dim) and differentiate through
the fused HIP backward kernels. Forward KL(B||A) is ``kl(b, a)``. Temperature,
its squared scaling, masking and normalisation stay with the caller, as the JSD
PR text on the pages states for all these per-token ops ("Changes").
"""

import torch

from . import binding as B


class _Logprobs(torch.autograd.Function):
    @staticmethod
    def forward(ctx, z, t, ignore_index, split_hint):
        logp, stats = B.logprobs_fwd(z, t, ignore_index, split_hint)
        ctx.save_for_backward(z, t, stats)
        ctx.ignore_index = ignore_index
        return logp

    @staticmethod
    def backward(ctx, g):
        z, t, stats = ctx.saved_tensors
        dz = B.logprobs_bwd(z, t, stats, g, ctx.ignore_index) if ctx.needs_input_grad[0] else None
        return dz, None, None, None


class _LogprobsTopk(torch.autograd.Function):
    @staticmethod
    def forward(ctx, z, ids, ignore_index, split_hint):
        logp, stats = B.logprobs_topk_fwd(z, ids, ignore_index, split_hint)
        ctx.save_for_backward(z, ids, stats)
        ctx.ignore_index = ignore_index
        return logp

    @staticmethod
    def backward(ctx, g):
        z, ids, stats = ctx.saved_tensors
        dz = B.logprobs_topk_bwd(z, ids, stats, g, ctx.ignore_index) if ctx.needs_input_grad[0] else None
        return dz, None, None, None


class _Entropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, z, split_hint):
        H, stats = B.entropy_fwd(z, split_hint)
        ctx.save_for_backward(z, stats, H)
        return H

    @staticmethod
    def backward(ctx, g):
        z, stats, H = ctx.saved_tensors
        return (B.entropy_bwd(z, stats, H, g) if ctx.needs_input_grad[0] else None), None


class _KL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, b, split_hint):
        kl, stats = B.kl_fwd(a, b, split_hint)
        ctx.save_for_backward(a, b, stats, kl)
        return kl

    @staticmethod
    def backward(ctx, g):
        a, b, stats, kl = ctx.saved_tensors
        na, nb = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (na or nb):
            return None, None, None
        da, db = B.kl_bwd(a, b, stats, kl, g, need_a=na, need_b=nb)
        return da, db, None


class _JSD(torch.autograd.Function):
    @staticmethod
    def forward(ctx, s, t, beta, split_hint):
        out, stats = B.jsd_fwd(s, t, beta, split_hint)
        ctx.save_for_backward(s, t, stats, out)
        ctx.beta = beta
        return out

    @staticmethod
    def backward(ctx, g):
        s, t, stats, out = ctx.saved_tensors
        ns, nt = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (ns or nt):
            return None, None, None, None
        ds, dt = B.jsd_bwd(s, t, ctx.beta, stats, out, g, need_s=ns, need_t=nt)
        return ds, dt, None, None


class _LinearLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, h, W, t, ignore_index, split_hint):
        logp, stats = B.linear_logp_fwd(h, W, t, ignore_index, split_hint)
        ctx.save_for_backward(h, W, t, stats)
        ctx.ignore_index = ignore_index
        return logp

    @staticmethod
    def backward(ctx, g):
        h, W, t, stats = ctx.saved_tensors
        nh, nw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (nh or nw):
            return None, None, None, None, None
        dh, dW = B.linear_logp_bwd(h, W, t, stats, g, ctx.ignore_index, need_h=nh, need_w=nw)
        return dh, dW, None, None, None


def linear_logp(h, W, t, ignore_index=-100, split_hint=0):
    """Per-token log p_t under logits h W^T, without materialising the logits (bf16 h, W).
    ``split_hint=SPLIT_INVARIANT`` (or any k >= 1) makes logp, and so dh, batch invariant."""
    return _LinearLogp.apply(h, W, t, ignore_index, split_hint)


def logprobs(z, t, ignore_index=-100, split_hint=0):
    """Per-token log p_t; ``t == ignore_index`` gives 0 and no gradient.

    ``t`` shaped like the logits without the last dim gives one value per row;
    ``t`` with an extra trailing dim K (top-k ids) gives [..., K] values, and the
    gradient adds the upstream gradients of duplicate ids.
    """
    if t.dim() == z.dim():
        return _LogprobsTopk.apply(z, t, ignore_index, split_hint)
    return _Logprobs.apply(z, t, ignore_index, split_hint)


def entropy(z, split_hint=0):
    """Per-token entropy -sum p log p."""
    return _Entropy.apply(z, split_hint)


def kl(a, b, split_hint=0):
    """Per-token KL(A||B) = sum p_A (log p_A - log p_B); +inf where B masks A's support."""
    return _KL.apply(a, b, split_hint)


def jsd(student, teacher, beta=0.5, split_hint=0):
    """Per-token generalized JSD with mixture M = (1 - beta) p_S + beta p_T:
    beta KL(T||M) + (1 - beta) KL(S||M); beta = 0 is KL(T||S), beta = 1 is KL(S||T)."""
    return _JSD.apply(student, teacher, float(beta), split_hint)
