"""The C ABI on the host: symbols, pure host queries, argument validation (no GPU needed).

Every call here either is a pure host function or fails validation before
anything is launched, so it runs without a device.
"""

import ctypes
import os
import re

import pytest

from vocab_wide_softmax_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vws.h")

EINVAL, EDTYPE, ELAYOUT, EWORKSPACE = -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"VWS_API\s+[\w\s\*]+?\b(vws_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert L.vws_version() == 103


def test_strerror(L):
    for s in (0, EINVAL, EDTYPE, ELAYOUT, EWORKSPACE, -5):
        assert len(B.strerror(s)) >= 2
    assert B.strerror(-99) == "unknown status"


def test_split_parts_and_workspace(L):
    # long rows, few of them: split; many rows: no split
    assert B.split_parts(B.OP_ENTROPY, 1024, 75968) == 1  # 1024 rows fill the chip unsplit
    assert B.split_parts(B.OP_ENTROPY, 256, 75968) == 3   # about 768 workgroups
    assert B.split_parts(B.OP_ENTROPY, 64, 75968) == 12
    assert B.split_parts(B.OP_ENTROPY, 1, 75968) == 18    # parts of at least 512 groups
    assert B.split_parts(B.OP_ENTROPY, 8192, 75968) == 1
    assert B.split_parts(B.OP_KL, 64, 1024, 4) == 4
    assert B.split_parts(B.OP_KL, 64, 1024, 16) == 16
    assert B.split_parts(B.OP_KL, 64, 1024, 1) == 1
    assert B.split_parts(B.OP_KL, 3, 20, 64) == 3  # capped at ceil(V/8) groups
    assert B.workspace_bytes(B.OP_ENTROPY, 8192, 75968) == 0
    assert B.workspace_bytes(B.OP_ENTROPY, 1024, 75968) == 0
    assert B.workspace_bytes(B.OP_ENTROPY, 256, 75968) == 256 * 3 * 3 * 4
    assert B.workspace_bytes(B.OP_KL, 256, 75968) == 256 * 3 * 6 * 4
    assert B.workspace_bytes(B.OP_KL, 1024, 75968, 8) == 1024 * 8 * 6 * 4
    assert B.workspace_bytes(B.OP_KL, 0, 75968) == 0
    with pytest.raises(ValueError):
        B.workspace_bytes(7, 10, 10)
    with pytest.raises(ValueError):
        B.workspace_bytes(B.OP_KL, 10, 0)


def _rows(data=0x1000, dtype=B.VWS_BF16, n_outer=4, n_inner=1, s_outer=64, s_inner=0, V=64, col_stride=1):
    return B.vws_rows(data, dtype, n_outer, n_inner, s_outer, s_inner, V, col_stride)


def _ent(L, r, out=0x2000, stats=0x3000, ws=None, nb=0, hint=0):
    return L.vws_entropy_fwd(ctypes.byref(r), out, stats, ws, nb, hint, None)


def test_forward_validation(L):
    assert _ent(L, _rows(dtype=5)) == EDTYPE
    assert _ent(L, _rows(V=0)) == EINVAL
    assert _ent(L, _rows(V=(1 << 31) - 1 - 4096 + 1, s_outer=1 << 31)) == EINVAL  # one past the widest row
    assert _ent(L, _rows(n_outer=-1)) == EINVAL
    assert _ent(L, _rows(col_stride=2)) == ELAYOUT
    assert _ent(L, _rows(s_outer=-64)) == ELAYOUT
    assert _ent(L, _rows(data=0x1001)) == ELAYOUT  # bf16 needs 2-byte alignment
    assert _ent(L, _rows(data=0)) == EINVAL
    assert _ent(L, _rows(), out=0) == EINVAL
    assert _ent(L, _rows(), stats=0) == EINVAL
    assert _ent(L, _rows(), out=0x2002) == ELAYOUT
    assert _ent(L, _rows(), hint=-2) == EINVAL
    assert _ent(L, _rows(s_outer=2 ** 62, n_outer=8)) == ELAYOUT  # address overflow
    # empty batch: no-op, even with null pointers
    assert _ent(L, _rows(n_outer=0, data=0), out=0, stats=0) == 0
    # workspace too small / missing when a split is requested
    assert _ent(L, _rows(V=4096, s_outer=4096), hint=4) == EWORKSPACE
    assert _ent(L, _rows(V=4096, s_outer=4096), ws=0x4000, nb=16, hint=4) == EWORKSPACE


def test_kl_and_logprobs_validation(L):
    a, b = _rows(), _rows(dtype=B.VWS_F32)
    assert L.vws_kl_fwd(ctypes.byref(a), ctypes.byref(b), 0x2000, 0x3000, None, 0, 0, None) == EDTYPE
    b = _rows(V=32, s_outer=32)
    assert L.vws_kl_fwd(ctypes.byref(a), ctypes.byref(b), 0x2000, 0x3000, None, 0, 0, None) == EINVAL
    b = _rows(n_outer=3)
    assert L.vws_kl_fwd(ctypes.byref(a), ctypes.byref(b), 0x2000, 0x3000, None, 0, 0, None) == EINVAL
    # kl backward with neither gradient requested is a no-op
    a = _rows()
    assert L.vws_kl_bwd(ctypes.byref(a), ctypes.byref(a), 0x3000, 0x2000, 0x5000, 1, None, None, None) == 0
    assert L.vws_kl_bwd(ctypes.byref(a), ctypes.byref(a), 0x3000, 0x2000, 0x5000, -1, 0x6000, None, None) == EINVAL
    t = B.vws_ids(0, 1, 0)
    assert L.vws_logprobs_fwd(ctypes.byref(a), ctypes.byref(t), -100, 0x2000, 0x3000, None, 0, 0, None) == EINVAL
    t = B.vws_ids(0x7004, 1, 0)  # int64 ids need 8-byte alignment
    assert L.vws_logprobs_fwd(ctypes.byref(a), ctypes.byref(t), -100, 0x2000, 0x3000, None, 0, 0, None) == ELAYOUT
    assert L.vws_logprobs_bwd(ctypes.byref(a), None, -100, 0x3000, 0x5000, 1, 0x6000, None) == EINVAL
    assert L.vws_entropy_bwd(ctypes.byref(a), 0x3000, 0, 0x5000, 1, 0x6000, None) == EINVAL  # H missing
    assert L.vws_entropy_bwd(ctypes.byref(a), 0x3000, 0x2000, 0x5000, 1, 0x6001, None) == ELAYOUT


def test_linear_validation(L):
    c_i64 = ctypes.c_int64

    def fwd(h=0x1000, ldh=64, W=0x2000, ldw=64, dtype=B.VWS_BF16, N=4, H=64, V=100, t=0x3000, logp=0x4000,
            stats=0x5000, ws=0x6000, nb=1 << 20, split=0):
        return L.vws_linear_logp_fwd(h, ldh, W, ldw, dtype, N, H, V, t, -100, logp, stats, ws, nb, split, None)

    assert fwd(dtype=B.VWS_F32) == EDTYPE
    assert fwd(H=0) == EINVAL
    assert fwd(ldh=60) == ELAYOUT  # row stride must be a multiple of 8 and >= H
    assert fwd(ldw=72, H=80) == ELAYOUT
    assert fwd(h=0x1008) == ELAYOUT  # 16-byte alignment
    assert fwd(t=0) == EINVAL
    assert fwd(logp=0) == EINVAL
    assert fwd(nb=16) == EWORKSPACE
    assert fwd(N=0, h=0, W=0, t=0) == 0
    # backward workspace: the dz pair (hi and lo planes of [N, chunk] bf16, 256-byte aligned), plus
    # the fp32 sum of dh [N, H] when the vocabulary spans more than one chunk of 8192 columns
    align = lambda x: (x + 255) // 256 * 256
    assert B.linear_workspace_bytes(1, 8, 64, 100) == 2 * align(8 * 104 * 2)
    assert B.linear_workspace_bytes(1, 8192, 4096, 151936) == 2 * 8192 * 8192 * 2 + 8192 * 4096 * 4
    assert B.linear_workspace_bytes(1, 8192, 4096, 151936) < 0.41e9
    assert B.linear_workspace_bytes(1, 300, 200, 3001, 3) == 2 * align(300 * 1024 * 2) + 300 * 200 * 4
    assert B.linear_workspace_bytes(1, 300, 200, 3001, 1) == 2 * align(300 * 3008 * 2)
    assert B.linear_workspace_bytes(0, 8, 64, 100) > 8 * 4
    with pytest.raises(ValueError):
        B.linear_workspace_bytes(2, 8, 64, 100)
    bwd = L.vws_linear_logp_bwd
    assert bwd(0x1000, 64, 0x2000, 64, B.VWS_BF16, 4, 64, 100, 0x3000, -100, 0x5000, 0x7000, -1, 0x8000, None, 0x6000,
               1 << 20, 0, None) == EINVAL
    assert bwd(0x1000, 64, 0x2000, 64, B.VWS_BF16, 4, 64, 100, 0x3000, -100, 0x5000, 0x7000, 1, 0x8000, None, 0x6000,
               1 << 20, -2, None) == EINVAL
    assert bwd(0x1000, 64, 0x2000, 64, B.VWS_BF16, 4, 64, 100, 0x3000, -100, 0x5000, 0x7000, 1, None, None, 0x6000,
               1 << 20, 0, None) == 0  # no gradient requested
    assert bwd(0x1000, 64, 0x2000, 64, B.VWS_BF16, 4, 64, 100, 0x3000, -100, 0x5000, 0x7000, 1, 0x8000, None, 0x6000,
               16, 0, None) == EWORKSPACE
    assert bwd(0x1000, 64, 0x2000, 64, B.VWS_BF16, 4, 64, 100, 0x3000, -100, 0x5000, 0x7000, 1, 0x8000, None, 0x6010,
               1 << 20, 0, None) == ELAYOUT  # the workspace is 256-byte aligned
    # more tiles than a launch of 512-thread workgroups can hold (2^23): rejected before any launch
    assert fwd(N=1 << 31, V=(1 << 31) - 1, nb=1 << 62) == EINVAL
    assert fwd(N=1 << 24, V=1 << 15, nb=1 << 62) == EINVAL  # 2^16 token x 2^7 vocabulary tiles
    assert fwd(N=1 << 31, V=100, nb=1 << 62) == EINVAL  # 2^23 token x 1 hidden tiles (dh)
    assert fwd(N=4, V=(1 << 31) - 1, nb=1 << 62) == EINVAL  # 2^23 vocabulary x 1 hidden tiles (dW)
    # forward chunking: split_hint below VWS_SPLIT_INVARIANT is invalid; the fixed modes size
    # the partials by V alone
    assert fwd(split=-2) == EINVAL
    with pytest.raises(ValueError):
        B.linear_workspace_bytes(0, 8, 64, 100, -2)
    per_row = lambda sp, v: (B.linear_workspace_bytes(0, 512, 64, v, sp) - 512 * 4) / (512 * 8)
    assert per_row(B.SPLIT_INVARIANT, 151936) == 149  # 594 vocabulary tiles in chunks of 4
    assert per_row(5, 151936) == 5
    assert B.linear_workspace_bytes(1, 8, 64, 100, B.SPLIT_INVARIANT) == 2 * align(8 * 104 * 2)


def test_topk_validation(L):
    a = _rows()

    def fwd(ids=0x7000, s_o=8, s_i=0, s_k=1, K=8, logp=0x2000, stats=0x3000, r=None):
        t = B.vws_ids_k(ids, s_o, s_i, s_k, K)
        r = r or a
        return L.vws_logprobs_topk_fwd(ctypes.byref(r), ctypes.byref(t), -100, logp, stats, None, 0, 0, None)

    def bwd(ids=0x7000, K=8, s_k=1, gr=8, gk=1, dz=0x6000, stats=0x3000):
        t = B.vws_ids_k(ids, 8, 0, s_k, K)
        return L.vws_logprobs_topk_bwd(ctypes.byref(a), ctypes.byref(t), -100, stats, 0x5000, gr, gk, dz, None)

    assert fwd(K=0) == EINVAL
    assert fwd(K=2049) == EINVAL
    assert fwd(ids=0) == EINVAL
    assert fwd(ids=0x7004) == ELAYOUT
    assert fwd(s_k=-1) == ELAYOUT
    assert fwd(logp=0) == EINVAL
    assert fwd(stats=0) == EINVAL
    assert fwd(logp=0x2002) == ELAYOUT
    assert fwd(r=_rows(n_outer=0, data=0), ids=0, logp=0, stats=0) == 0  # empty batch
    assert bwd(K=0) == EINVAL
    assert bwd(gr=-1) == EINVAL
    assert bwd(gk=-1) == EINVAL
    assert bwd(dz=0) == EINVAL
    assert bwd(dz=0x6001) == ELAYOUT
    assert bwd(stats=0) == EINVAL


def test_jsd_validation(L):
    s, t = _rows(), _rows()
    f = ctypes.c_float

    def fwd(beta=0.5, jsd=0x2000, stats=0x3000, ws=0x4000, nb=1 << 20, a=None, b=None):
        return L.vws_jsd_fwd(ctypes.byref(a or s), ctypes.byref(b or t), f(beta), jsd, stats, ws, nb, 0, None)

    assert fwd(beta=-0.1) == EINVAL
    assert fwd(beta=1.5) == EINVAL
    assert fwd(beta=float("nan")) == EINVAL
    assert fwd(b=_rows(dtype=B.VWS_F32)) == EDTYPE
    assert fwd(b=_rows(V=32, s_outer=32)) == EINVAL
    assert fwd(jsd=0) == EINVAL
    assert fwd(stats=0x3002) == ELAYOUT
    assert fwd(ws=None, nb=0) == EWORKSPACE
    assert fwd(nb=16) == EWORKSPACE
    assert fwd(a=_rows(n_outer=0, data=0), b=_rows(n_outer=0, data=0), jsd=0, stats=0, ws=None, nb=0) == 0
    assert B.workspace_bytes(B.OP_JSD, 8, 100) == 8 * 4 * 4
    assert B.workspace_bytes(B.OP_JSD, 4, 151936) == 4 * 4 * 4 + 4 * B.split_parts(B.OP_JSD, 4, 151936) * 8 * 4
    # the endpoints are the KL calls: their argument errors are the KL ones
    assert fwd(beta=0.0, b=_rows(dtype=B.VWS_F32)) == EDTYPE
    assert fwd(beta=1.0, jsd=0) == EINVAL
    bw = L.vws_jsd_bwd
    assert bw(ctypes.byref(s), ctypes.byref(t), f(0.5), 0x3000, 0x2000, 0x5000, -1, 0x6000, None, None) == EINVAL
    assert bw(ctypes.byref(s), ctypes.byref(t), f(0.5), 0, 0x2000, 0x5000, 1, 0x6000, None, None) == EINVAL
    assert bw(ctypes.byref(s), ctypes.byref(t), f(0.5), 0x3000, 0x2000, 0x5000, 1, None, None, None) == 0
    assert bw(ctypes.byref(s), ctypes.byref(t), f(0.5), 0x3000, 0x2000, 0x5000, 1, 0x6001, None, None) == ELAYOUT


def test_batch_invariant_split_depends_on_v_only(L):
    for V, want in ((1024, 1), (32768, 1), (32769, 2), (75968, 3), (151936, 5)):
        got = {B.split_parts(op, n, V, B.SPLIT_INVARIANT) for op in (0, 1, 2, 3) for n in (1, 7, 64, 1024, 8192)}
        assert got == {want}, (V, got)
    # the automatic choice does depend on N (that is what the invariant mode avoids)
    assert B.split_parts(0, 64, 75968) != B.split_parts(0, 8192, 75968)
    assert B.workspace_bytes(2, 8192, 75968, B.SPLIT_INVARIANT) == 8192 * 3 * 6 * 4
    assert L.vws_split_parts(0, 8, 100, -2) < 0


def test_binding_rejects_host_tensors():
    """The Python binding refuses host tensors before any pointer reaches the library."""
    import torch

    z = torch.zeros(4, 16, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int64)
    ids = torch.zeros(4, 3, dtype=torch.int64)
    st2, st4, st6 = torch.zeros(4, 2), torch.zeros(4, 4), torch.zeros(4, 6)
    g, v = torch.ones(4), torch.zeros(4)
    h, W = torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(16, 8, dtype=torch.bfloat16)
    calls = [
        lambda: B.logprobs_fwd(z, t),
        lambda: B.logprobs_bwd(z, t, st2, g),
        lambda: B.logprobs_topk_fwd(z, ids),
        lambda: B.logprobs_topk_bwd(z, ids, st2, torch.ones(4, 3)),
        lambda: B.entropy_fwd(z),
        lambda: B.entropy_bwd(z, st2, v, g),
        lambda: B.kl_fwd(z, z),
        lambda: B.kl_bwd(z, z, st4, v, g),
        lambda: B.jsd_fwd(z, z, 0.5),
        lambda: B.jsd_bwd(z, z, 0.5, st6, v, g),
        lambda: B.linear_logp_fwd(h, W, t),
        lambda: B.linear_logp_bwd(h, W, t, st2, g),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU tensors"):
            call()


def test_missing_library_fails_loudly(monkeypatch):
    """Without libvws.so every entry point raises: there is no CPU or PyTorch fallback."""
    import torch

    monkeypatch.setattr(B, "_LIB_PATH", os.path.join(ROOT, "no_such_dir", "libvws.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        B.lib()
    if torch.cuda.is_available():  # on a GPU machine the call itself must raise too
        z = torch.zeros(4, 16, dtype=torch.bfloat16, device="cuda:0")
        with pytest.raises(ImportError):
            B.entropy_fwd(z)


def test_kl_fwd_noalloc_validation(L):
    """The allocation-free KL forward validates like vws_kl_fwd and rejects, before any launch,
    a split whose partial states exceed the static scratch."""
    a, b = _rows(), _rows(dtype=B.VWS_F32)
    f = L.vws_kl_fwd_noalloc
    assert f(ctypes.byref(a), ctypes.byref(b), 0x2000, 0x3000, 0, None) == EDTYPE
    assert f(ctypes.byref(a), ctypes.byref(a), 0, 0x3000, 0, None) == EINVAL
    assert f(ctypes.byref(a), ctypes.byref(a), 0x2000, 0x3000, -2, None) == EINVAL
    e = _rows(n_outer=0, data=0)
    assert f(ctypes.byref(e), ctypes.byref(e), 0, 0, 0, None) == 0  # empty batch
    # 8192 rows x 64 parts x 6 floats = 12.6 MB of partial states > 8 MiB
    big = _rows(n_outer=8192, V=75968, s_outer=75968)
    need = B.workspace_bytes(B.OP_KL, 8192, 75968, 64)
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), ctypes.byref(big), 0x2000, 0x3000, 64, None) == -6
    assert "static scratch" in B.strerror(-6)
