"""GPU parity of the fused linear-logp (MFMA) against the fp64 oracle, through the C ABI.

Every comparison uses the standard rule of oracle.compare (fp32 outputs within 2e-5
relative or 64 eps32 c; bf16 gradients within one bf16 ulp of the oracle's RNE value or
that plus 64 eps32 c; NaN / inf positions equal), with the worst error-to-allowance
ratio asserted <= 1 and the strict misses printed:

* small ragged shape (300 tokens, hidden 200, vocabulary 3000: partial tiles in
  every dimension, ignored targets): every element of logp, lse, dh and dW, in one
  backward chunk and forced into 3 chunks (the fp32 dh sum's first, middle and last
  steps, a last chunk whose width is not a multiple of 8);
* the dz pair itself: after a one-chunk backward the workspace holds hi and lo of every
  dz entry; hi passes the bf16 rule against the oracle's dz and hi + lo the fp32 rule;
* degenerate shapes: one token, a one-column vocabulary, hidden size 8;
* an out-of-range target: NaN logp and dh row, NaN dW (the row's dz is NaN);
* the full hidden and vocabulary widths (4096 x 151936) at 512 tokens: every
  logp and dh element, sampled dW rows;
* the full 8192 x 4096 x 151936 launch (slow): sampled rows of logp and dh,
  sampled vocabulary rows of dW, targeted and untargeted;
* 8548 tokens x vocabulary 16684 (34 token tiles, 66 vocabulary tiles): every
  element, with every branch of the forward's and the dz pass's block-to-tile
  orders in use (whole groups and the tiles past them in both dimensions), in the
  automatic chunking and in one chunk;
* the batch-invariant forward chunkings (fixed 1024-column chunks, and a fixed
  chunk count): every element against the oracle, and sub-batches whose logp,
  stats and dh equal the full batch's rows bit for bit;
* a chunk's dW and dh as one grid (4096 x 2304 x 8192) against each gradient alone:
  the same bits;
* the two tile heights of dz and dh (256 tokens, and 128 where 256 would fill at
  most half of the CUs; every smaller case above takes 128): sub-batches on the
  other side of the switch give the full batch's dh bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import compare, linear_logp as OL
from vocab_wide_softmax_amd import binding as B
from vocab_wide_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _assert_ok(rep, label):
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, (label, rep)
    assert rep["worst"] <= 1.0, (label, rep)
    print(label, {k: (rep[k] if not isinstance(rep[k], float) else round(rep[k], 4)) for k in rep}, flush=True)


def _small(n=300, hidden=200, v=3000, seed=11):
    gen = torch.Generator().manual_seed(seed)
    h = torch.randn(n, hidden, generator=gen).to(torch.bfloat16)
    Wm = (0.05 * torch.randn(v, hidden, generator=gen)).to(torch.bfloat16)
    t = torch.randint(0, v, (n,), generator=gen)
    t[::37] = -100
    g = torch.randn(n, generator=gen)
    return h, Wm, t, g


def _run(h, Wm, t, g, device, need_h=True, need_w=True, split=0, bsplit=0, ws=None):
    dh_, Wd, td, gd = h.to(device), Wm.to(device), t.to(device), g.to(device)
    logp, stats = B.linear_logp_fwd(dh_, Wd, td, -100, split)
    dh, dW = B.linear_logp_bwd(dh_, Wd, td, stats, gd, -100, need_h=need_h, need_w=need_w, split_hint=bsplit, ws=ws)
    torch.cuda.synchronize()
    return logp, stats, dh, dW


@pytest.mark.parametrize("bsplit,v", [(0, 3000), (3, 3001)])
def test_linear_small_all_elements(device, bsplit, v):
    h, Wm, t, g = _small(v=v)
    logp, stats, dh, dW = _run(h, Wm, t, g, device, bsplit=bsplit)
    hh, hw, ht, hg = f64(h), f64(Wm), t.numpy(), g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    c = OL.cond_linear_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, c, "f32"), "small logp")
    lse_dev = f64(stats[:, 0]) + f64(stats[:, 1])
    _assert_ok(compare.check(lse_dev, m + ls, c, "f32"), "small lse")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "small dh")
    _assert_ok(compare.check(f64(dW), OL.linear_logp_bwd_dw(hh, hw, ht, hg), OL.cond_linear_dw(hh, hw, ht, hg),
                             "bf16"), "small dW")


def test_linear_dz_pair_pin(device):
    """One backward chunk leaves the whole dz pair in the workspace: hi = rne(dz) holds every
    element to the bf16 rule against the oracle's dz = g (onehot(t) - p) of the fp64 logits,
    and hi + lo to the fp32 rule (the pair carries dz to about 2^-17)."""
    h, Wm, t, g = _small(n=300, hidden=200, v=3000, seed=13)
    n, v = 300, 3000
    nb = B.linear_workspace_bytes(1, n, 200, v)
    ldc = (v + 7) // 8 * 8
    plane = (n * ldc * 2 + 255) // 256 * 256
    assert nb == 2 * plane  # one chunk: no fp32 dh sum
    ws = torch.zeros(nb, dtype=torch.uint8, device=device)
    _run(h, Wm, t, g, device, ws=ws)
    hi = ws[:n * ldc * 2].view(torch.bfloat16).view(n, ldc)
    lo = ws[plane:plane + n * ldc * 2].view(torch.bfloat16).view(n, ldc)
    assert torch.count_nonzero(hi[:, v:]) == 0 and torch.count_nonzero(lo[:, v:]) == 0  # zero padding
    hh, hw, ht, hg = f64(h), f64(Wm), t.numpy(), g.double().numpy()
    dz = OL.linear_logp_bwd_dz(hh, hw, ht, hg)
    c = OL.cond_linear_dz(hh, hw, ht, hg)
    _assert_ok(compare.check(f64(hi[:, :v]), dz, c, "bf16"), "dz hi")
    _assert_ok(compare.check(f64(hi[:, :v]) + f64(lo[:, :v]), dz, c, "f32"), "dz hi+lo")


def test_linear_out_of_range_target(device):
    h, Wm, t, g = _small(n=40, hidden=64, v=500, seed=3)
    t[5] = 500
    logp, stats, dh, dW = _run(h, Wm, t, g, device)
    lp = logp.cpu()
    assert torch.isnan(lp[5]) and not torch.isnan(lp[torch.arange(40) != 5]).any()
    assert torch.isnan(dh[5].float()).all() and not torch.isnan(dh[6].float()).any()
    assert torch.isnan(dW.float()).all()
    assert (lp[t == -100] == 0).all()


def test_linear_gradient_subsets(device):
    h, Wm, t, g = _small(n=64, hidden=96, v=700, seed=5)
    _, _, dh_both, dW_both = _run(h, Wm, t, g, device)
    _, _, dh_only, none_w = _run(h, Wm, t, g, device, need_w=False)
    _, _, none_h, dW_only = _run(h, Wm, t, g, device, need_h=False)
    assert none_w is None and none_h is None
    assert torch.equal(dh_both, dh_only) and torch.equal(dW_both, dW_only)


def test_linear_grouped_dw_dh_grid_keeps_bits(device):
    """4096 tokens, hidden 2304, vocabulary 8192: one chunk of 32 vocabulary tiles x 9 hidden
    tiles (288 dW blocks, a multiple of 8) and 16 x 9 token tiles for dh (above the small-batch
    switch), so a backward asking for both gradients runs them as one grid (dW tiles, then dh
    tiles); asking for one at a time runs each alone. Both must give the same bits, and sampled
    rows of both gradients must match the oracle."""
    gen = torch.Generator().manual_seed(21)
    h = torch.randn(4096, 2304, generator=gen).to(torch.bfloat16)
    Wm = (0.03 * torch.randn(8192, 2304, generator=gen)).to(torch.bfloat16)
    t = torch.randint(0, 8192, (4096,), generator=gen)
    t[::53] = -100
    g = torch.randn(4096, generator=gen)
    _, _, dh_both, dW_both = _run(h, Wm, t, g, device)
    _, _, dh_only, _ = _run(h, Wm, t, g, device, need_w=False)
    _, _, _, dW_only = _run(h, Wm, t, g, device, need_h=False)
    assert torch.equal(dh_both, dh_only) and torch.equal(dW_both, dW_only)
    hh, hw, ht, hg = f64(h), f64(Wm), t.numpy(), g.double().numpy()
    rows = np.array([0, 1, 777, 2048, 4095])
    _assert_ok(compare.check(f64(dh_both[torch.from_numpy(rows).to(device)]),
                             OL.linear_logp_bwd_dh(hh, hw, ht, hg, rows=rows),
                             OL.cond_linear_dh(hh, hw, ht, hg, rows=rows), "bf16"), "grouped dh rows")
    cols = np.unique(np.concatenate([ht[ht >= 0][:6], [0, 255, 256, 4097, 8191]]))
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg, vocab_rows=cols)
    _assert_ok(compare.check(f64(dW_both[torch.from_numpy(cols).to(device)]), dw_ref, dw_c, "bf16"),
               "grouped dW rows")


def test_linear_full_width_512_tokens(device):
    wl = W.linear_logp(n=512, seed=4)
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    c = OL.cond_linear_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, c, "f32"), "512 logp")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "512 dh")
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([ht[:8], rng.integers(0, hw.shape[0], 40), [0, hw.shape[0] - 1]]))
    dw_ref, dw_c = OL.linear_logp_bwd_dw(hh, hw, ht, hg, vocab_rows=cols), OL.cond_linear_dw(hh, hw, ht, hg,
                                                                                              vocab_rows=cols)
    _assert_ok(compare.check(f64(dW[torch.from_numpy(cols).to(dW.device)]), dw_ref, dw_c, "bf16"),
               "512 dW rows")


@pytest.mark.slow
def test_linear_full_size_sampled(device):
    wl = W.linear_logp()
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, hh.shape[0] - 1], rng.integers(0, hh.shape[0], 14)]))
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht, rows=rows)
    c = OL.cond_linear_fwd(hh, hw, ht, rows=rows)
    idx = torch.from_numpy(rows).to(device)
    _assert_ok(compare.check(f64(logp[idx]), lp, c, "f32"), "full logp rows")
    _assert_ok(compare.check(f64(dh[idx]), OL.linear_logp_bwd_dh(hh, hw, ht, hg, rows=rows),
                             OL.cond_linear_dh(hh, hw, ht, hg, rows=rows), "bf16"), "full dh rows")
    # dW: 64 targeted and 192 untargeted vocabulary rows, including each backward chunk's first
    # and last rows (chunks of 8192 columns)
    edges = np.concatenate([np.arange(0, hw.shape[0], 8192), np.arange(8191, hw.shape[0], 8192), [hw.shape[0] - 1]])
    untargeted = np.setdiff1d(np.arange(hw.shape[0]), ht)
    cols = np.unique(np.concatenate([ht[:64], rng.choice(untargeted, 192, replace=False), edges]))
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg, vocab_rows=cols)
    _assert_ok(compare.check(f64(dW[torch.from_numpy(cols).to(device)]), dw_ref, dw_c, "bf16"),
               "full dW rows")


@pytest.mark.slow
@pytest.mark.parametrize("bsplit", [0, 1])
def test_linear_tile_orders_all_elements(device, bsplit):
    """34 token tiles (four whole super-tiles of 8 plus 2, the last partial; one whole group of
    32 for the forward) and 66 vocabulary tiles (backward: chunks of 32, 32 and 2 tiles, or one
    chunk of two whole 32-tile super-tiles plus 2, the last partial): a tile the block orders
    skipped or visited twice would leave a wrong logp, dh or dW element."""
    wl = W.linear_logp(n=8548, hidden=128, v=16684, seed=9, w_std=0.1)
    wl.t[::97] = -100
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device, bsplit=bsplit)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    for r0 in range(0, hh.shape[0], 1024):
        rows = np.arange(r0, min(r0 + 1024, hh.shape[0]))
        lp, m, ls = OL.linear_logp_fwd(hh, hw, ht, rows=rows)
        c = OL.cond_linear_fwd(hh, hw, ht, rows=rows)
        _assert_ok(compare.check(f64(logp[r0:rows[-1] + 1]), lp, c, "f32"), "orders logp %d" % r0)
        lse_dev = f64(stats[r0:rows[-1] + 1, 0]) + f64(stats[r0:rows[-1] + 1, 1])
        _assert_ok(compare.check(lse_dev, m + ls, c, "f32"), "orders lse %d" % r0)
        _assert_ok(compare.check(f64(dh[r0:rows[-1] + 1]), OL.linear_logp_bwd_dh(hh, hw, ht, hg, rows=rows),
                                 OL.cond_linear_dh(hh, hw, ht, hg, rows=rows), "bf16"),
                   "orders dh %d" % r0)
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg)
    _assert_ok(compare.check(f64(dW), dw_ref, dw_c, "bf16"), "orders dW")


@pytest.mark.parametrize("n,hidden,v", [(1, 8, 1), (3, 8, 1), (1, 8, 7), (2, 16, 300)])
def test_linear_degenerate_shapes(device, n, hidden, v):
    """One token, a one-column vocabulary (logp 0, zero gradients: p = 1 at the target) and the
    smallest hidden size; every element against the oracle."""
    gen = torch.Generator().manual_seed(n * 1000 + v)
    h = torch.randn(n, hidden, generator=gen).to(torch.bfloat16)
    Wm = (0.3 * torch.randn(v, hidden, generator=gen)).to(torch.bfloat16)
    t = torch.randint(0, v, (n,), generator=gen)
    g = torch.randn(n, generator=gen)
    logp, stats, dh, dW = _run(h, Wm, t, g, device)
    hh, hw, ht, hg = f64(h), f64(Wm), t.numpy(), g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    c = OL.cond_linear_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, c, "f32"), "degenerate logp")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "degenerate dh")
    _assert_ok(compare.check(f64(dW), OL.linear_logp_bwd_dw(hh, hw, ht, hg), OL.cond_linear_dw(hh, hw, ht, hg),
                             "bf16"), "degenerate dW")
    if v == 1:
        assert (logp.cpu() == 0).all()
        assert torch.count_nonzero(dh) == 0 and torch.count_nonzero(dW) == 0


@pytest.mark.parametrize("split", [B.SPLIT_INVARIANT, 3])
def test_linear_batch_invariant(device, split):
    """Fixed vocabulary chunking (depending on V alone): 600 tokens (three token tiles, the last
    ragged) over a 5000-column vocabulary, then sub-batches cut at other offsets; logp, stats and
    dh of each sub-batch row must be the full batch's bits."""
    h, Wm, t, g = _small(n=600, hidden=128, v=5000, seed=17)
    logp, stats, dh, dW = _run(h, Wm, t, g, device, split=split)
    hh, hw, ht, hg = f64(h), f64(Wm), t.numpy(), g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    c = OL.cond_linear_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, c, "f32"), "invariant logp")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "invariant dh")
    _assert_ok(compare.check(f64(dW), OL.linear_logp_bwd_dw(hh, hw, ht, hg), OL.cond_linear_dw(hh, hw, ht, hg),
                             "bf16"), "invariant dW")
    for r0, r1 in ((0, 37), (300, 301), (513, 600)):
        lp_s, st_s, dh_s, _ = _run(h[r0:r1], Wm, t[r0:r1], g[r0:r1], device, need_w=False, split=split)
        assert torch.equal(lp_s, logp[r0:r1]), (split, r0, r1)
        assert torch.equal(st_s, stats[r0:r1]), (split, r0, r1)
        assert torch.equal(dh_s.view(torch.int16), dh[r0:r1].view(torch.int16)), (split, r0, r1)


def test_linear_tile_height_keeps_dh_bits(device):
    """dz and dh take 128-token tiles where 256-token ones would fill at most half of the CUs. The
    8448-token batch at H = 1024 takes 256-token tiles for dh and for the dz of its two whole
    8192-column chunks (128-token ones for the 300-column last chunk); its 1000- and 517-token
    sub-batches take 128-token tiles throughout. With the batch-invariant forward, each
    sub-batch's logp, stats and dh rows must be the full batch's bits: the tile height changes
    neither a token row's place in its MFMA block nor any entry's k-sequence."""
    h, Wm, t, g = _small(n=8448, hidden=1024, v=16684, seed=23)
    logp, stats, dh, _ = _run(h, Wm, t, g, device, need_w=False, split=B.SPLIT_INVARIANT)
    for r0, r1 in ((0, 1000), (4000, 4517)):
        print("tile height", r0, r1, flush=True)
        lp_s, st_s, dh_s, _ = _run(h[r0:r1], Wm, t[r0:r1], g[r0:r1], device, need_w=False, split=B.SPLIT_INVARIANT)
        assert torch.equal(lp_s, logp[r0:r1]), (r0, r1)
        assert torch.equal(st_s, stats[r0:r1]), (r0, r1)
        assert torch.equal(dh_s.view(torch.int16), dh[r0:r1].view(torch.int16)), (r0, r1)


def test_linear_strided_rows_broadcast_g_and_partial_stage(device):
    """Row pitches above H (views of wider buffers), H = 72 (a partial last k-stage), ragged
    N and V (partial tiles in both), and an upstream gradient broadcast from one value."""
    gen = torch.Generator().manual_seed(21)
    n, hidden, v = 257, 72, 1000
    hb = torch.randn(n, 88, generator=gen).to(torch.bfloat16)
    wb = (0.08 * torch.randn(v, 80, generator=gen)).to(torch.bfloat16)
    t = torch.randint(0, v, (n,), generator=gen)
    t[::50] = -100
    h_dev, w_dev = hb.to(device)[:, :hidden], wb.to(device)[:, :hidden]
    assert h_dev.stride(0) == 88 and w_dev.stride(0) == 80
    g = torch.tensor(0.625)
    logp, stats = B.linear_logp_fwd(h_dev, w_dev, t.to(device), -100)
    dh, dW = B.linear_logp_bwd(h_dev, w_dev, t.to(device), stats, g.to(device).expand(n), -100, split_hint=2)
    torch.cuda.synchronize()
    hh, hw, ht = f64(hb[:, :hidden]), f64(wb[:, :hidden]), t.numpy()
    hg = np.full(n, 0.625)
    _assert_ok(compare.check(f64(logp), OL.linear_logp_fwd(hh, hw, ht)[0], OL.cond_linear_fwd(hh, hw, ht), "f32"),
               "strided logp")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "strided dh")
    _assert_ok(compare.check(f64(dW), OL.linear_logp_bwd_dw(hh, hw, ht, hg), OL.cond_linear_dw(hh, hw, ht, hg),
                             "bf16"), "strided dW")


@pytest.mark.parametrize("n,hidden,v", [(256, 64, 512), (256, 128, 512), (256, 192, 768),
                                         (32, 256, 512), (64, 256, 512), (96, 256, 512)])
def test_linear_short_reductions_all_elements(device, n, hidden, v):
    """Interior tiles with one to three k-stages: the forward's ping-pong loop at hidden 64 / 128 /
    192 (64-deep stages) and the dW pair's at 32 / 64 / 96 tokens (32-deep stages), where the
    prologue issues fewer stages than the ring holds and the in-flight counts of the waits are
    smallest; all elements against the oracle."""
    wl = W.linear_logp(n=n, hidden=hidden, v=v, seed=31 + n + hidden, w_std=0.1)
    wl.t[::7] = -100
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, OL.cond_linear_fwd(hh, hw, ht), "f32"), "short logp %d %d" % (n, hidden))
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "short dh %d %d" % (n, hidden))
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg)
    _assert_ok(compare.check(f64(dW), dw_ref, dw_c, "bf16"), "short dW %d %d" % (n, hidden))


def test_linear_multichunk_interior_all_elements(device):
    """512 tokens, hidden 512 and three vocabulary chunks of 8192: every dh tile is interior and
    takes, chunk by chunk, the first / add / last epilogue of the fp32 running sum (batched reads,
    paired bf16 rounding), every dW and dz tile the interior epilogue; all elements against the
    oracle."""
    wl = W.linear_logp(n=512, hidden=512, v=3 * 8192, seed=29, w_std=0.05)
    wl.t[::41] = -100
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, OL.cond_linear_fwd(hh, hw, ht), "f32"), "multichunk logp")
    _assert_ok(compare.check(f64(dh), OL.linear_logp_bwd_dh(hh, hw, ht, hg), OL.cond_linear_dh(hh, hw, ht, hg),
                             "bf16"), "multichunk dh")
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg)
    _assert_ok(compare.check(f64(dW), dw_ref, dw_c, "bf16"), "multichunk dW")


@pytest.mark.slow
def test_linear_xcd_patch_orders_all_elements(device):
    """Hidden width 4096 (16 hidden tiles) with 17 token tiles and 17 vocabulary tiles: the dh and
    dW contractions map their first 16 x 16 tiles through the XCD patch order and the last row of
    tiles in row-major order; a tile visited twice or never would leave a wrong dh or dW element."""
    wl = W.linear_logp(n=4352, hidden=4096, v=4200, seed=23, w_std=0.02)
    wl.t[::89] = -100
    logp, stats, dh, dW = _run(wl.h, wl.W, wl.t, wl.g, device)
    hh, hw, ht, hg = f64(wl.h), f64(wl.W), wl.t.numpy(), wl.g.double().numpy()
    lp, m, ls = OL.linear_logp_fwd(hh, hw, ht)
    _assert_ok(compare.check(f64(logp), lp, OL.cond_linear_fwd(hh, hw, ht), "f32"), "patch logp")
    for r0 in range(0, hh.shape[0], 1088):
        rows = np.arange(r0, min(r0 + 1088, hh.shape[0]))
        _assert_ok(compare.check(f64(dh[r0:rows[-1] + 1]), OL.linear_logp_bwd_dh(hh, hw, ht, hg, rows=rows),
                                 OL.cond_linear_dh(hh, hw, ht, hg, rows=rows), "bf16"), "patch dh %d" % r0)
    dw_ref, dw_c = OL.linear_logp_bwd_dw_cond(hh, hw, ht, hg)
    _assert_ok(compare.check(f64(dW), dw_ref, dw_c, "bf16"), "patch dW")
