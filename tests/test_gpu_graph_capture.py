"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on ROCm).

The C ABI enqueues kernels only (no allocation, no synchronisation, no memset
nodes), so a whole forward + backward step can be captured once and replayed.
Each replay, with unrelated eager work and synchronisations in between, must
reproduce the eager results bit for bit: logprobs (split path), entropy, KL
with both gradients, top-k logprobs, JSD and the fused linear-logp.
"""

import pytest
import torch

from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu


def _inputs(device):
    gen = torch.Generator().manual_seed(17)
    a = (3.0 * torch.randn(96, 3000, generator=gen)).bfloat16().to(device)
    b = (a.float().cpu() + 0.5 * torch.randn(96, 3000, generator=gen)).bfloat16().to(device)
    t = torch.randint(0, 3000, (96,), generator=gen).to(device)
    ids = torch.randint(0, 3000, (96, 5), generator=gen).to(device)
    g = torch.randn(96, generator=gen).to(device)
    gk = torch.randn(96, 5, generator=gen).to(device)
    h = torch.randn(64, 96, generator=gen).bfloat16().to(device)
    W = (0.1 * torch.randn(900, 96, generator=gen)).bfloat16().to(device)
    tl = torch.randint(0, 900, (64,), generator=gen).to(device)
    gl = torch.randn(64, generator=gen).to(device)
    return a, b, t, ids, g, gk, h, W, tl, gl


def _step(a, b, t, ids, g, gk, h, W, tl, gl):
    out = []
    lp, st = B.logprobs_fwd(a, t, -100, 4)  # forced split: partials + combine kernel
    out += [lp, st, B.logprobs_bwd(a, t, st, g, -100)]
    H, st = B.entropy_fwd(a)
    out += [H, B.entropy_bwd(a, st, H, g)]
    kl, st = B.kl_fwd(a, b)
    out += [kl, *B.kl_bwd(a, b, st, kl, g)]
    lk, st = B.logprobs_topk_fwd(a, ids, -100)
    out += [lk, B.logprobs_topk_bwd(a, ids, st, gk, -100)]
    jo, st = B.jsd_fwd(a, b, 0.3)
    out += [jo, *B.jsd_bwd(a, b, 0.3, st, jo, g)]
    ll, st = B.linear_logp_fwd(h, W, tl)
    out += [ll, *B.linear_logp_bwd(h, W, tl, st, gl)]
    return out


def _bits(x):
    return x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)


def test_graph_replays_match_eager(device):
    args = _inputs(device)
    eager = [x.clone() for x in _step(*args)]
    torch.cuda.synchronize()
    # warm up on a side stream (allocator state), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(*args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(*args)
    for rep in range(3):
        # unrelated eager work between replays
        scratch = torch.randn(1 << 20, device=device).sum()
        torch.cuda.synchronize()
        for x in captured:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        graph.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(captured, eager)):
            assert torch.equal(_bits(x), _bits(y)), (rep, i)
        del scratch
