"""The allocation-free KL forward (vws_kl_fwd_noalloc) against vws_kl_fwd, through the C ABI.

It must give the same bits as the workspace entry point with the same split_hint (the
same kernels, with the split's partial states in the library's static per-GPU scratch),
on two calls in a row whose second is smaller (leftover partial states of the first call
must not leak into it), and pass the fp64 oracle's rule.
"""

import numpy as np
import pytest
import torch

from oracle import compare, reductions as R
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu


def _pair(n, v, seed):
    gen = torch.Generator().manual_seed(seed)
    a = 3.0 * torch.randn(n, v, generator=gen)
    b = a + 0.5 * torch.randn(n, v, generator=gen)
    a[0] += 1e4
    b[0] += 1e4
    b[1, torch.randperm(v, generator=gen)[:16]] = -float("inf")
    return a.to(torch.bfloat16), b.to(torch.bfloat16)


@pytest.mark.parametrize("calls", [((512, 20000, 0), (64, 3000, 7)), ((1024, 75968, 8), (96, 40000, B.SPLIT_INVARIANT))])
def test_noalloc_matches_workspace_entry(device, calls):
    for i, (n, v, split) in enumerate(calls):
        print("noalloc call", i, "n", n, "v", v, "split", split, flush=True)
        a, b = _pair(n, v, seed=100 + i)
        assert B.split_parts(B.OP_KL, n, v, split) > 1  # the scratch is in use
        need = B.workspace_bytes(B.OP_KL, n, v, split)
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
        ad, bd = a.to(device), b.to(device)
        kl_ref, st_ref = B.kl_fwd(ad, bd, split)
        kl, st = B.kl_fwd_noalloc(ad, bd, split)
        torch.cuda.synchronize()
        assert torch.equal(kl.view(torch.int32), kl_ref.view(torch.int32)), (n, v, split)
        assert torch.equal(st.view(torch.int32), st_ref.view(torch.int32)), (n, v, split)
        ha, hb = a.double().numpy(), b.double().numpy()
        rows = np.arange(min(n, 48))
        y, _ = R.kl_fwd(ha[rows], hb[rows])
        rep = compare.check(kl[:len(rows)].double().cpu().numpy(), y, R.cond_kl_fwd(ha[rows], hb[rows]), "f32")
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
        assert np.isposinf(kl[1].item())  # row 1: B masks columns A supports


def test_noalloc_rejects_oversized_split(device):
    a, b = _pair(8192, 1024, seed=7)
    ad, bd = a.to(device), b.to(device)
    assert B.workspace_bytes(B.OP_KL, 8192, 1024, 128) > B.NOALLOC_SCRATCH_BYTES
    with pytest.raises(B.VwsError, match="static scratch"):
        B.kl_fwd_noalloc(ad, bd, 128)
    kl, _ = B.kl_fwd_noalloc(ad, bd, 1)  # no split: no scratch needed
    kl_ref, _ = B.kl_fwd(ad, bd, 1)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl_ref)
