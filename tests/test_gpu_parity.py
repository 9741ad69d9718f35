"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Workloads (vocab_wide_softmax_amd.workloads):
* tiny      64 x 1024 fp32 pair (row 0 offset +1e4, row 1 with 16 masked B
            columns): every element, all four ops, forward and backward, with
            the automatic launch and with the vocabulary forced into 4 and 16
            parts (the in-GPU combine).
* pair1024  1024 x 75968 bf16 pair (5% rows +1e4, 1% rows with 64 masked B
            columns): every element of every output and gradient; the
            automatic launch splits the vocabulary here.
* pair8192  8192 x 75968 bf16 pair: the full launch the benchmark times,
            checked on sampled rows (row 0, offset rows, masked rows, random),
            for the four ops (bf16 and the fp16 rounding of the pair) and for
            top-k logprobs (K = 16) and the JSD.
* shifted   [4, 2049, 75968] fp32 pair read through base[:, :-1, :]: the full
            in-place strided launch, checked on sampled rows.
"""

import numpy as np
import pytest
import torch

from parity import OPS, check_parity, f64, run_device, run_oracle
from vocab_wide_softmax_amd import binding as B
from vocab_wide_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


def _host_inputs(wl):
    a, b, t = wl.views()
    return f64(a.reshape(-1, a.shape[-1])), f64(b.reshape(-1, b.shape[-1])), t.reshape(-1).numpy()


def _to_device(wl, device):
    a_base = wl.a_base.to(device)
    b_base = wl.b_base.to(device)
    ids_base = wl.ids_base.to(device)
    a, b, t = wl.views(a_base, b_base, ids_base)
    return a, b, t


@pytest.fixture(scope="module")
def tiny(device):
    wl = W.workload("tiny")
    return wl, _to_device(wl, device), _host_inputs(wl)


@pytest.mark.parametrize("split", [0, 4, 16])
@pytest.mark.parametrize("op", OPS)
def test_tiny_all_elements(tiny, op, split):
    wl, (a, b, t), (ha, hb, ht) = tiny
    g = wl.g[op]
    print("tiny", op, "split", split, flush=True)
    dev = run_device(op, a, b, t, g.to(a.device), split_hint=split)
    ora = run_oracle(op, ha, hb, ht, g.double().numpy())
    check_parity(dev, ora, "f32", "tiny %s split %d" % (op, split))


@pytest.fixture(scope="module")
def pair1024(device):
    wl = W.workload("pair1024")
    return wl, _to_device(wl, device), _host_inputs(wl)


@pytest.mark.parametrize("op", OPS)
def test_pair1024_all_elements(pair1024, op):
    """Every element at 1024 x 75968, in the automatic launch (unsplit at this row count) and with
    the vocabulary split into 8 parts merged by the in-GPU combine."""
    wl, (a, b, t), (ha, hb, ht) = pair1024
    assert B.split_parts(B.OP_KL, a.shape[0], a.shape[1]) == 1
    assert B.split_parts(B.OP_KL, a.shape[0], a.shape[1], 8) == 8
    ora = run_oracle(op, ha, hb, ht, wl.g[op].double().numpy())
    for split in (0, 8):
        print("pair1024", op, "split", split, flush=True)
        dev = run_device(op, a, b, t, wl.g[op].to(a.device), split_hint=split)
        reps = check_parity(dev, ora, "bf16", "pair1024 %s split %d" % (op, split))
        print({k: (v["strict_miss"], round(v["worst"], 3)) for k, v in reps.items()}, flush=True)
        del dev


def _sample_rows(wl, n, k=24, seed=5):
    rng = np.random.default_rng(seed)
    rows = {0, n - 1}
    rows.update(wl.offset_rows[:8].tolist())
    rows.update(wl.mask_rows[:8].tolist())
    rows.update(rng.choice(n, size=k, replace=False).tolist())
    return np.array(sorted(rows))


def _sampled_parity(wl, device, ops, grad_kind):
    a, b, t = _to_device(wl, device)
    n = a.shape[0] if a.dim() == 2 else a.shape[0] * a.shape[1]
    rows = _sample_rows(wl, n)
    ha_all, hb_all, ht_all = wl.views()
    V = ha_all.shape[-1]
    ha = f64(ha_all.reshape(-1, V)[rows]) if not wl.shifted else f64(ha_all.reshape(n, V)[rows])
    hb = f64(hb_all.reshape(-1, V)[rows]) if not wl.shifted else f64(hb_all.reshape(n, V)[rows])
    ht = ht_all.reshape(-1)[rows].numpy()
    idx = torch.from_numpy(rows).to(device)
    for op in ops:
        print(wl.name, op, flush=True)
        g = wl.g[op]
        full = run_device_sampled(op, a, b, t, g.to(device), idx)
        ora = run_oracle(op, ha, hb, ht, g.double().numpy()[rows])
        check_parity(full, ora, grad_kind, "%s %s" % (wl.name, op))
        torch.cuda.empty_cache()


def run_device_sampled(op, a, b, t, g, idx):
    """Run the full launch, keep only the sampled rows (gathered on the device)."""
    res = {}
    if op == "logprobs":
        out, stats = B.logprobs_fwd(a, t, -100)
        grads = (B.logprobs_bwd(a, t, stats, g, -100),)
    elif op == "entropy":
        out, stats = B.entropy_fwd(a)
        grads = (B.entropy_bwd(a, stats, out, g),)
    else:
        x, y = (a, b) if op == "kl_ab" else (b, a)
        out, stats = B.kl_fwd(x, y)
        grads = B.kl_bwd(x, y, stats, out, g)
    V = a.shape[-1]
    res["out"] = f64(out.reshape(-1)[idx])
    res["stats"] = f64(stats[idx])
    res["grads"] = [f64(d.reshape(-1, V)[idx]) for d in grads]
    del grads, out, stats
    return res


@pytest.fixture(scope="module")
def pair8192():
    return W.workload("pair8192")


@pytest.mark.slow
def test_pair8192_sampled_rows(device, pair8192):
    _sampled_parity(pair8192, device, OPS, "bf16")


@pytest.mark.slow
def test_pair8192_fp16_sampled_rows(device, pair8192):
    """The same pair rounded to fp16, as in the benchmark's fp16 step (8192-row launch)."""
    import dataclasses

    wl = dataclasses.replace(pair8192, name="pair8192_fp16", a_base=pair8192.a_base.half(),
                             b_base=pair8192.b_base.half())
    _sampled_parity(wl, device, OPS, "f16")


@pytest.mark.slow
def test_pair8192_topk_and_jsd_sampled_rows(device, pair8192):
    """Top-k logprobs (K = 16) and the JSD at beta = 0.5 in the launch the benchmark times
    (8192 rows: one workgroup per row, no vocabulary split), the same seeded ids and
    upstream gradients, checked against the oracle on sampled rows."""
    from oracle import compare, jsd as J, topk as TK

    wl = pair8192
    a, b, _ = _to_device(wl, device)
    n, V = a.shape
    assert B.split_parts(B.OP_LOGPROBS, n, V) == 1 and B.split_parts(B.OP_JSD, n, V) == 1
    rows = _sample_rows(wl, n)
    idx = torch.from_numpy(rows).to(device)
    ids = torch.randint(0, V, (n, 16), generator=torch.Generator().manual_seed(5))
    ids[rows[1], 3] = ids[rows[1], 2]  # a duplicate id in a sampled row
    ids[rows[2], :] = -100  # a fully ignored sampled row
    gk = torch.randn(n, 16, generator=torch.Generator().manual_seed(6))
    trows = torch.from_numpy(rows)
    ha, hb = f64(wl.a[trows]), f64(wl.b[trows])
    print("pair8192 topk16", flush=True)
    di, dg = ids.to(device), gk.to(device)
    lp, st = B.logprobs_topk_fwd(a, di, -100)
    dz = B.logprobs_topk_bwd(a, di, st, dg, -100)
    hi, hg = ids.numpy()[rows], gk.double().numpy()[rows]
    rep = compare.check(f64(lp[idx]), TK.logprobs_topk_fwd(ha, hi)[0], TK.cond_logprobs_topk_fwd(ha, hi), "f32")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    rep = compare.check(f64(dz[idx]), TK.logprobs_topk_bwd(ha, hi, hg), TK.cond_logprobs_topk_bwd(ha, hi, hg), "bf16")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    del dz, lp, st
    print("pair8192 jsd0.5", flush=True)
    g = wl.g["kl_ab"]
    out, st = B.jsd_fwd(a, b, 0.5)
    ds, dt = B.jsd_bwd(a, b, 0.5, st, out, g.to(device))
    hgj = g.double().numpy()[rows]
    rep = compare.check(f64(out[idx]), J.jsd_fwd(ha, hb, 0.5)[0], J.cond_jsd_fwd(ha, hb, 0.5), "f32")
    assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    rs, rt = J.jsd_bwd(ha, hb, hgj, 0.5)
    cs, ct = J.cond_jsd_bwd(ha, hb, hgj, 0.5)
    for x, y, c in ((ds, rs, cs), (dt, rt, ct)):
        rep = compare.check(f64(x[idx]), y, c, "bf16")
        assert rep["fail"] == 0 and rep["nan_mismatch"] == 0 and rep["inf_mismatch"] == 0, rep
    del ds, dt, out, st
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def shifted():
    return W.workload("shifted")


@pytest.mark.slow
def test_shifted_fp32_sampled_rows(device, shifted):
    wl = shifted
    a, _, _ = wl.views()
    assert not a.is_contiguous()
    _sampled_parity(wl, device, ("entropy", "kl_ab", "logprobs"), "f32")


@pytest.mark.slow
def test_shifted_fp32_reads_in_place(device, shifted):
    """The causal-shift view is read in place (the second commit message of PR #8838 reads
    logits[:, :-1] through two row strides instead of copying it): with the two fp32 bases
    resident, the peak device memory of each op's forward + backward grows by no more than
    its outputs, statistics, gradients and workspace plus 1 MiB, so nothing copies the
    2.49 GB view (the pages report extra peak memory below 1 MiB)."""
    wl = shifted
    ab, bb, ib = wl.a_base.to(device), wl.b_base.to(device), wl.ids_base.to(device)
    a, b, t = wl.views(ab, bb, ib)
    assert not a.is_contiguous() and a.data_ptr() == ab.data_ptr()
    n, V = a.shape[0] * a.shape[1], a.shape[-1]
    for op in ("entropy", "kl_ab", "logprobs"):
        g = wl.g[op].to(device)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        if op == "entropy":
            out, st = B.entropy_fwd(a)
            grads = (B.entropy_bwd(a, st, out, g),)
            ws = B.workspace_bytes(B.OP_ENTROPY, n, V)
        elif op == "logprobs":
            out, st = B.logprobs_fwd(a, t, -100)
            grads = (B.logprobs_bwd(a, t, st, g, -100),)
            ws = B.workspace_bytes(B.OP_LOGPROBS, n, V)
        else:
            out, st = B.kl_fwd(a, b)
            grads = B.kl_bwd(a, b, st, out, g)
            ws = B.workspace_bytes(B.OP_KL, n, V)
        torch.cuda.synchronize()
        growth = torch.cuda.max_memory_allocated() - base
        need = sum(x.numel() * x.element_size() for x in grads) + out.numel() * 4 + st.numel() * 4 + ws
        assert all(x.is_contiguous() and x.dtype == torch.float32 for x in grads)
        print(op, "peak growth", growth, "outputs + gradients + workspace", need, flush=True)
        assert growth <= need + (1 << 20), (op, growth, need)
        del out, st, grads
    del ab, bb, ib, a, b, t
    torch.cuda.empty_cache()
