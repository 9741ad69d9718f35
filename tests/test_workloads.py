"""The seeded input generators: determinism and the stated structure (CPU only)."""

import torch

from vocab_wide_softmax_amd import workloads as W


def test_tiny_pair_structure_and_determinism():
    w1, w2 = W.workload("tiny"), W.workload("tiny")
    assert torch.equal(w1.a, w2.a) and torch.equal(w1.b, w2.b) and torch.equal(w1.t, w2.t)
    assert w1.a.shape == (64, 1024) and w1.a.dtype == torch.float32
    assert w1.a[0].min() > 9000 and w1.b[0].min() > 9000
    assert int(torch.isneginf(w1.b[1]).sum()) == 16
    assert int(torch.isneginf(w1.b).sum()) == 16 and not torch.isinf(w1.a).any()
    assert (w1.t >= 0).all() and (w1.t < 1024).all()
    assert set(w1.g) == set(W.OPS)


def test_logit_pair_recipe_small():
    w = W.logit_pair(200, v=3000, seed=7)
    assert w.a.dtype == torch.bfloat16 and w.a.shape == (200, 3000)
    assert len(w.offset_rows) == 10 and len(w.mask_rows) == 2 and 0 in w.offset_rows and 0 in w.mask_rows
    off = w.a.float()[w.offset_rows]
    assert off.min() > 9000
    for r in w.mask_rows.tolist():
        assert int(torch.isneginf(w.b[r]).sum()) == 64
    others = torch.ones(200, dtype=torch.bool)
    others[w.mask_rows] = False
    assert not torch.isinf(w.b[others]).any()
    # B is A plus small noise on unmasked, unoffset entries
    plain = torch.ones(200, dtype=torch.bool)
    plain[w.offset_rows] = False
    plain[w.mask_rows] = False
    d = (w.b.float() - w.a.float())[plain]
    assert 0.4 < float(d.std()) < 0.6
    w2 = W.logit_pair(200, v=3000, seed=7)
    assert torch.equal(w.a, w2.a) and torch.equal(w.b, w2.b)


def test_shifted_pair_is_a_view_without_copy():
    w = W.shifted_pair(batch=2, seq=5, v=64, seed=3)
    a, b, t = w.views()
    assert a.shape == (2, 4, 64) and a.data_ptr() == w.a_base.data_ptr()
    assert a.stride() == (5 * 64, 64, 1)
    assert t.shape == (2, 4) and t.stride() == (5, 1)
    assert torch.equal(t, w.ids_base[:, 1:])
