"""The largest inputs the library accepts, on the GPU: the widest rows (against oracle.grouped)
and the most rows (against the dense oracle).

V = INT32_MAX - 4096 = 2147479551 columns (4.3 GB per bf16 row) is the largest vocabulary the
C ABI takes (column and group indexes are 32-bit). Rows this wide cannot be held on the host as
float64, so each row is made of a few distinct values and one large repeated bulk, and the
count-weighted forms of oracle.grouped (pinned against the dense oracle on the CPU) give every
output and every gradient entry:

* recipe 0: bulk 0.0 in both inputs; columns 0 and 1 hold other values, column V/2 is -inf
  in both, and the row maximum sits in the last column (a pass that stopped short of the end
  would miss it). The bulk carries almost all of the probability, so S sums 2^31 equal terms.
* recipe 1: bulk -inf (masked) in both inputs with four live columns, the last one included.

Layouts: one row at the limit (16-byte loads, ragged last group), two rows at the limit (odd
row pitch: the element-wise path) and two rows at V - 7 (a multiple of 8: 16-byte loads in
every row). Each runs logprobs, entropy, KL(A||B), KL(B||A), the generalized JSD at beta = 0.5
and top-k logprobs (K = 3 with a duplicate id, and K = 65 with ids in the last column tile)
forward and backward, in the automatic and the batch-invariant split. Forward
values and the special columns' gradients are compared with the grouped forms under the parity
rule; every bulk gradient entry is checked at once: the number of entries equal to the bulk's
value must be the bulk's size (plus the special columns that share that value), and that value
must meet the rule too.

Most rows: N = INT32_MAX rows of V = 8 columns (one backward tile per row, the most the
backward grid takes), cycling through three row patterns. The first three rows are compared
with the dense oracle under the parity rule; every other row's output, statistics and gradient
must equal, bit for bit, those of the first row with the same pattern (each row is reduced by
the same code in the same order, wherever it sits).
"""

import numpy as np
import pytest
import torch

from oracle import compare, grouped as Gr, reductions as R
from vocab_wide_softmax_amd import binding as B

pytestmark = pytest.mark.gpu
VMAX = 2**31 - 1 - 4096
NINF = float("-inf")
IGN = -100


def _recipe(k, V):
    """(special columns, a values, b values, bulk a, bulk b, target column, top-k columns)."""
    if k == 0:
        cols = [0, 1, V // 2, V - 1]
        return cols, [2.0, 0.0, NINF, 8.0], [0.0, 1.0, NINF, 4.0], 0.0, 0.0, V - 1, [V - 1, 0, V - 1]
    cols = [0, 12345, V // 3, V - 1]
    return cols, [1.0, 0.5, 2.0, 3.0], [0.0, 1.0, 1.5, 2.5], NINF, NINF, V // 3, [V // 3, 12345, 0]


def _groups(k, V):
    cols, av, bv, ab, bb, t, tk = _recipe(k, V)
    a = np.array(av + [ab])
    b = np.array(bv + [bb])
    cnt = np.array([1] * len(cols) + [V - len(cols)], dtype=np.int64)
    return a, b, cnt, cols.index(t), [cols.index(c) for c in tk]


def _build(n, V, device):
    a = torch.empty(n, V, dtype=torch.bfloat16, device=device)
    b = torch.empty(n, V, dtype=torch.bfloat16, device=device)
    t = torch.empty(n, dtype=torch.int64)
    ids = torch.empty(n, 3, dtype=torch.int64)
    for r in range(n):
        cols, av, bv, ab, bb, tc, tk = _recipe(r, V)
        a[r].fill_(ab)
        b[r].fill_(bb)
        idx = torch.tensor(cols, device=device)
        a[r, idx] = torch.tensor(av, dtype=torch.bfloat16, device=device)
        b[r, idx] = torch.tensor(bv, dtype=torch.bfloat16, device=device)
        t[r] = tc
        ids[r] = torch.tensor(tk)
    return a, b, t.to(device), ids.to(device)


def _ok(rep, label):
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, (label, rep)


def _check_fwd(dev, ref, cond, label):
    _ok(compare.check(dev.detach().double().cpu().numpy(), np.asarray(ref, dtype=np.float64),
                      np.asarray(cond, dtype=np.float64), "f32"), label)


def _check_grad(d, r, V, grad, cond, label):
    """d [n, V] bf16 gradient on the device, grad / cond per group of row r (specials, then bulk)."""
    cols = _recipe(r, V)[0]
    bulk_col = 2 if r == 0 else 1  # a bulk column in either recipe
    spec = d[r, torch.tensor(cols, device=d.device)]
    bulk = d[r, bulk_col]
    same = int((d[r] == bulk).sum().item())
    shared = int((spec == bulk).sum().item())
    assert same == (V - len(cols)) + shared, (label, same, V - len(cols), shared)
    vals = torch.cat([spec, bulk.reshape(1)]).double().cpu().numpy()
    _ok(compare.check(vals, np.asarray(grad, dtype=np.float64), np.asarray(cond, dtype=np.float64), "bf16"), label)


@pytest.mark.slow
@pytest.mark.parametrize("n,V", [(1, VMAX), (2, VMAX), (2, VMAX - 7)], ids=["one-row-max", "two-rows-max", "two-rows-aligned"])
@pytest.mark.parametrize("split", [0, B.SPLIT_INVARIANT], ids=["auto", "invariant"])
def test_max_vocab(device, n, V, split):
    print("max vocab n", n, "V", V, "split", split, flush=True)
    a, b, t, ids = _build(n, V, device)
    g = torch.tensor([0.75, -1.5][:n], device=device)
    gk = torch.tensor([[0.5, -1.25, 2.0], [1.0, 0.25, -0.5]][:n], device=device)
    G = [_groups(r, V) for r in range(n)]

    lp, st = B.logprobs_fwd(a, t, IGN, split)
    _check_fwd(lp, [Gr.logprobs_fwd(x[0], x[2], x[3])[0] for x in G], [Gr.cond_logprobs_fwd(x[0], x[2], x[3]) for x in G],
               "logprobs fwd")
    d = B.logprobs_bwd(a, t, st, g, IGN)
    for r, (ga, gb, cnt, tg, _) in enumerate(G):
        _check_grad(d, r, V, Gr.logprobs_bwd(ga, cnt, tg, g[r].item()), Gr.cond_logprobs_bwd(ga, cnt, tg, g[r].item()),
                    "logprobs bwd row %d" % r)
    del d

    H, st = B.entropy_fwd(a, split)
    _check_fwd(H, [Gr.entropy_fwd(x[0], x[2])[0] for x in G], [Gr.cond_entropy_fwd(x[0], x[2]) for x in G], "entropy fwd")
    d = B.entropy_bwd(a, st, H, g)
    for r, (ga, gb, cnt, _, _) in enumerate(G):
        _check_grad(d, r, V, Gr.entropy_bwd(ga, cnt, g[r].item()), Gr.cond_entropy_bwd(ga, cnt, g[r].item()),
                    "entropy bwd row %d" % r)
    del d

    for x, y, sw in ((a, b, False), (b, a, True)):
        name = "KL(B||A)" if sw else "KL(A||B)"
        kl, st = B.kl_fwd(x, y, split)
        refs = [Gr.kl_fwd(gb, ga, cnt)[0] if sw else Gr.kl_fwd(ga, gb, cnt)[0] for ga, gb, cnt, _, _ in G]
        conds = [Gr.cond_kl_fwd(gb, ga, cnt) if sw else Gr.cond_kl_fwd(ga, gb, cnt) for ga, gb, cnt, _, _ in G]
        _check_fwd(kl, refs, conds, name + " fwd")
        dx, dy = B.kl_bwd(x, y, st, kl, g)
        for r, (ga, gb, cnt, _, _) in enumerate(G):
            gx, gy = (gb, ga) if sw else (ga, gb)
            rx, ry = Gr.kl_bwd(gx, gy, cnt, g[r].item())
            cx, cy = Gr.cond_kl_bwd(gx, gy, cnt, g[r].item())
            _check_grad(dx, r, V, rx, cx, "%s bwd first row %d" % (name, r))
            _check_grad(dy, r, V, ry, cy, "%s bwd second row %d" % (name, r))
        del dx, dy

    # generalized JSD at beta = 0.5 (student A, teacher B)
    jv, st = B.jsd_fwd(a, b, 0.5, split)
    _check_fwd(jv, [Gr.jsd_fwd(ga, gb, cnt, 0.5)[0] for ga, gb, cnt, _, _ in G],
               [Gr.cond_jsd_fwd(ga, gb, cnt, 0.5) for ga, gb, cnt, _, _ in G], "jsd fwd")
    ds, dt = B.jsd_bwd(a, b, 0.5, st, jv, g)
    for r, (ga, gb, cnt, _, _) in enumerate(G):
        rs, rt = Gr.jsd_bwd(ga, gb, cnt, g[r].item(), 0.5)
        cs, ct = Gr.cond_jsd_bwd(ga, gb, cnt, g[r].item(), 0.5)
        _check_grad(ds, r, V, rs, cs, "jsd bwd student row %d" % r)
        _check_grad(dt, r, V, rt, ct, "jsd bwd teacher row %d" % r)
    del ds, dt

    out, st = B.logprobs_topk_fwd(a, ids, IGN, split)
    for r, (ga, gb, cnt, _, sl) in enumerate(G):
        _check_fwd(out[r], Gr.logprobs_topk_fwd(ga, cnt, sl)[0], Gr.cond_logprobs_topk_fwd(ga, cnt, sl),
                   "topk fwd row %d" % r)
    d = B.logprobs_topk_bwd(a, ids, st, gk, IGN)
    for r, (ga, gb, cnt, _, sl) in enumerate(G):
        gr = gk[r].double().cpu().numpy()
        _check_grad(d, r, V, Gr.logprobs_topk_bwd(ga, cnt, sl, gr), Gr.cond_logprobs_topk_bwd(ga, cnt, sl, gr),
                    "topk bwd row %d" % r)
    del d

    # K = 65 runs the slot kernel with LDS (8192-column tiles): 33 slots name the last column,
    # whose tile ends past INT32_MAX at the limit, and 32 name column 0
    ids65 = torch.tensor([[V - 1] * 33 + [0] * 32] * n, device=device)
    gk65 = torch.linspace(-1.0, 1.5, 65 * n, device=device).reshape(n, 65)
    out, st = B.logprobs_topk_fwd(a, ids65, IGN, split)
    d = B.logprobs_topk_bwd(a, ids65, st, gk65, IGN)
    for r, (ga, gb, cnt, _, _) in enumerate(G):
        sl = [3] * 33 + [0] * 32  # groups of columns V - 1 and 0 in either recipe
        gr = gk65[r].double().cpu().numpy()
        _check_fwd(out[r], Gr.logprobs_topk_fwd(ga, cnt, sl)[0], Gr.cond_logprobs_topk_fwd(ga, cnt, sl),
                   "topk65 fwd row %d" % r)
        _check_grad(d, r, V, Gr.logprobs_topk_bwd(ga, cnt, sl, gr), Gr.cond_logprobs_topk_bwd(ga, cnt, sl, gr),
                    "topk65 bwd row %d" % r)
    del d, a, b
    torch.cuda.empty_cache()


def _same_as_pattern(x, P, label):
    """Every row of x [N, ...] equals row (r mod P) of x bit for bit."""
    N = x.shape[0]
    flat = x.reshape(N, -1)
    bits = flat.view(torch.int16) if flat.element_size() == 2 else flat.view(torch.int32)
    head = bits[:P]
    M = (N // P) * P
    step = P * (1 << 22)
    for c in range(0, M, step):
        e = min(M, c + step)
        blk = bits[c:e].reshape(-1, P, bits.shape[1])
        assert torch.equal(blk, head.unsqueeze(0).expand_as(blk)), (label, c)
    assert torch.equal(bits[M:], head[: N - M]), (label, "tail")


@pytest.mark.slow
def test_max_rows(device):
    N, V, P = 2**31 - 1, 8, 3
    print("max rows N", N, "V", V, flush=True)
    pats = torch.tensor([[0.5, -1.0, 2.0, 0.0, 1.5, -3.0, 0.25, 1.0],
                         [NINF, 4.0, 3.0, NINF, -2.0, 3.5, 0.0, 1.0],
                         [1e4, 1e4 + 8, 1e4 - 8, 1e4, 1e4 + 16, 1e4, 1e4 - 16, 1e4 + 8]]).bfloat16()
    tpat = torch.tensor([2, 5, 4])
    reps = N // P + 1
    a = pats.to(device).repeat(reps, 1)[:N]
    t = tpat.to(device).repeat(reps)[:N]
    g = torch.tensor(0.75, device=device).expand(N)
    z3, t3, g3 = pats.double().numpy(), tpat.numpy(), np.full(P, 0.75)

    lp, st = B.logprobs_fwd(a, t, IGN)
    ref, _, _ = R.logprobs_fwd(z3, t3, IGN)
    _check_fwd(lp[:P], ref, R.cond_logprobs_fwd(z3, t3, IGN), "max rows logprobs fwd")
    _same_as_pattern(lp, P, "logprobs out")
    _same_as_pattern(st, P, "logprobs stats")
    d = B.logprobs_bwd(a, t, st, g, IGN)
    _ok(compare.check(d[:P].double().cpu().numpy(), R.logprobs_bwd(z3, t3, g3, IGN),
                      R.cond_logprobs_bwd(z3, t3, g3, IGN), "bf16"), "max rows logprobs bwd")
    _same_as_pattern(d, P, "logprobs grad")
    del d, lp, st

    H, st = B.entropy_fwd(a)
    _check_fwd(H[:P], R.entropy_fwd(z3)[0], R.cond_entropy_fwd(z3), "max rows entropy fwd")
    _same_as_pattern(H, P, "entropy out")
    d = B.entropy_bwd(a, st, H, g)
    _ok(compare.check(d[:P].double().cpu().numpy(), R.entropy_bwd(z3, g3), R.cond_entropy_bwd(z3, g3), "bf16"),
        "max rows entropy bwd")
    _same_as_pattern(d, P, "entropy grad")
    del d, H, st, a, t
    torch.cuda.empty_cache()
