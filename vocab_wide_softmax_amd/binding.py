"""ctypes binding of libvws (include/vws.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of libvws.so; this
module turns torch tensors into the C descriptors, allocates outputs (torch
owns device memory), passes torch's current HIP stream of the tensors' GPU
(with that GPU made current for the call), and raises ``VwsError`` on a
non-zero status. Tensors on the host or on different GPUs raise ValueError
before any pointer reaches the library. There is no fallback: if libvws.so is
missing or fails to load, the first call raises.

Layouts: logits are [N, V] or [B, S, V] tensors whose last dimension is
contiguous; the leading dimensions are passed as (at most) two row strides,
so a view like ``logits[:, :-1, :]`` is read in place. Targets and upstream
gradients have the shape of the logits without the last dimension.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvws.so")

VWS_F32, VWS_BF16, VWS_F16 = 0, 1, 2
OP_LOGPROBS, OP_ENTROPY, OP_KL, OP_JSD = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 8 << 20  # VWS_NOALLOC_SCRATCH_BYTES of vws.h
SPLIT_INVARIANT = -1  # fixed V-only vocabulary segments: results independent of the batch
_DTYPES = {torch.float32: VWS_F32, torch.bfloat16: VWS_BF16, torch.float16: VWS_F16}


class VwsError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed with status %d: %s" % (fn, status, msg))
        self.status = status


class vws_rows(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("n_outer", ctypes.c_int64),
        ("n_inner", ctypes.c_int64),
        ("s_outer", ctypes.c_int64),
        ("s_inner", ctypes.c_int64),
        ("V", ctypes.c_int64),
        ("col_stride", ctypes.c_int64),
    ]


class vws_ids(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("s_outer", ctypes.c_int64), ("s_inner", ctypes.c_int64)]


class vws_ids_k(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("s_outer", ctypes.c_int64), ("s_inner", ctypes.c_int64),
                ("s_k", ctypes.c_int64), ("K", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded libvws.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libvws.so not built at %s (run python -m vocab_wide_softmax_amd.build)" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, SZ, VP, FP = (ctypes.POINTER, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p)
        R, T, TK = P(vws_rows), P(vws_ids), P(vws_ids_k)
        sig = {
            "vws_workspace_bytes": (SZ, [I32, I64, I64, I32]),
            "vws_split_parts": (I32, [I32, I64, I64, I32]),
            "vws_logprobs_fwd": (I32, [R, T, I64, FP, FP, VP, SZ, I32, VP]),
            "vws_logprobs_bwd": (I32, [R, T, I64, FP, FP, I64, VP, VP]),
            "vws_logprobs_topk_fwd": (I32, [R, TK, I64, FP, FP, VP, SZ, I32, VP]),
            "vws_logprobs_topk_bwd": (I32, [R, TK, I64, FP, FP, I64, I64, VP, VP]),
            "vws_entropy_fwd": (I32, [R, FP, FP, VP, SZ, I32, VP]),
            "vws_entropy_bwd": (I32, [R, FP, FP, FP, I64, VP, VP]),
            "vws_kl_fwd": (I32, [R, R, FP, FP, VP, SZ, I32, VP]),
            "vws_kl_fwd_noalloc": (I32, [R, R, FP, FP, I32, VP]),
            "vws_kl_bwd": (I32, [R, R, FP, FP, FP, I64, VP, VP, VP]),
            "vws_jsd_fwd": (I32, [R, R, ctypes.c_float, FP, FP, VP, SZ, I32, VP]),
            "vws_jsd_bwd": (I32, [R, R, ctypes.c_float, FP, FP, FP, I64, VP, VP, VP]),
            "vws_linear_workspace_bytes": (SZ, [I32, I64, I64, I64, I32]),
            "vws_linear_logp_fwd": (I32, [VP, I64, VP, I64, I32, I64, I64, I64, VP, I64, FP, FP, VP, SZ, I32, VP]),
            "vws_linear_logp_bwd": (I32, [VP, I64, VP, I64, I32, I64, I64, I64, VP, I64, FP, FP, I64, VP, VP, VP,
                                          SZ, I32, VP]),
            "vws_strerror": (ctypes.c_char_p, [I32]),
            "vws_version": (I32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def library_path():
    return _LIB_PATH


def strerror(status):
    return lib().vws_strerror(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise VwsError(fn, status, strerror(status))


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def rows(t: torch.Tensor) -> vws_rows:
    """Descriptor of a [N, V] or [B, S, V] logits tensor (last dim contiguous)."""
    if t.dtype not in _DTYPES:
        raise TypeError("logits must be float32, bfloat16 or float16, got %s" % t.dtype)
    if t.dim() == 2:
        n_outer, n_inner, s_outer, s_inner = t.shape[0], 1, t.stride(0), 0
    elif t.dim() == 3:
        n_outer, n_inner, s_outer, s_inner = t.shape[0], t.shape[1], t.stride(0), t.stride(1)
    else:
        raise ValueError("logits must be 2-D [N, V] or 3-D [B, S, V]")
    col_stride = t.stride(-1) if t.shape[-1] > 1 else 1
    return vws_rows(t.data_ptr(), _DTYPES[t.dtype], n_outer, n_inner, s_outer, s_inner, t.shape[-1], col_stride)


def ids(t: torch.Tensor, like: torch.Tensor) -> vws_ids:
    """Descriptor of int64 targets shaped like ``like`` without its last dim."""
    if t.dtype != torch.int64:
        raise TypeError("targets must be int64")
    if tuple(t.shape) != tuple(like.shape[:-1]):
        raise ValueError("targets shape %s does not match logits %s" % (tuple(t.shape), tuple(like.shape)))
    if t.dim() == 1:
        return vws_ids(t.data_ptr(), t.stride(0), 0)
    return vws_ids(t.data_ptr(), t.stride(0), t.stride(1))


def ids_k(t: torch.Tensor, like: torch.Tensor) -> vws_ids_k:
    """Descriptor of int64 ids shaped like ``like`` with its last dim replaced by K."""
    if t.dtype != torch.int64:
        raise TypeError("ids must be int64")
    if t.dim() != like.dim() or tuple(t.shape[:-1]) != tuple(like.shape[:-1]):
        raise ValueError("ids shape %s does not match logits %s" % (tuple(t.shape), tuple(like.shape)))
    if t.dim() == 2:
        return vws_ids_k(t.data_ptr(), t.stride(0), 0, t.stride(1), t.shape[1])
    return vws_ids_k(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2), t.shape[2])


def _n_rows(z):
    n = 1
    for s in z.shape[:-1]:
        n *= s
    return n


def _g_arg(g: torch.Tensor, like: torch.Tensor):
    """(tensor, stride) for the fp32 upstream gradient: flat stride 1 or 0 (broadcast)."""
    if g.dtype != torch.float32:
        g = g.float()
    if g.numel() == 1 or all(s == 0 for s in g.stride()):
        return g, 0
    g = g.reshape(-1)
    if g.numel() != _n_rows(like):
        raise ValueError("upstream gradient has %d elements, expected %d" % (g.numel(), _n_rows(like)))
    if g.stride(0) != 1:
        g = g.contiguous()
    return g, 1


def _outputs(z, k):
    n = _n_rows(z)
    out = torch.empty(z.shape[:-1], dtype=torch.float32, device=z.device)
    stats = torch.empty((n, k), dtype=torch.float32, device=z.device)
    return out, stats


def workspace_bytes(op, n, v, split_hint=0):
    r = lib().vws_workspace_bytes(op, n, v, split_hint)
    if r == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace query")
    return r


def split_parts(op, n, v, split_hint=0):
    return lib().vws_split_parts(op, n, v, split_hint)


def _workspace(op, z, split_hint):
    nbytes = workspace_bytes(op, _n_rows(z), z.shape[-1], split_hint)
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=z.device), nbytes


def _ptr(t):
    return None if t is None else t.data_ptr()


def _device(*tensors):
    """The one GPU every given tensor lives on. Host tensors are rejected here, before any
    pointer reaches the library (a host pointer in a kernel would be a memory fault)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libvws takes GPU tensors; got a tensor on %s" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))
    return dev


# ------------------------------------------------------------------- entry points

def logprobs_fwd(z, t, ignore_index=-100, split_hint=0):
    """(logp fp32 [N...], stats fp32 [N, 2]) -- vws_logprobs_fwd."""
    dev = _device(z, t)
    L = lib()
    logp, stats = _outputs(z, 2)
    ws, nb = _workspace(OP_LOGPROBS, z, split_hint)
    r, ti = rows(z), ids(t, z)
    with torch.cuda.device(dev):
        _check("vws_logprobs_fwd", L.vws_logprobs_fwd(ctypes.byref(r), ctypes.byref(ti), ignore_index, _ptr(logp),
                                                      _ptr(stats), _ptr(ws), nb, split_hint, _stream(dev)))
    return logp, stats


def logprobs_bwd(z, t, stats, g, ignore_index=-100):
    """dz [shape of z, contiguous, dtype of z] -- vws_logprobs_bwd."""
    dev = _device(z, t, stats, g)
    L = lib()
    g, gs = _g_arg(g, z)
    dz = torch.empty(z.shape, dtype=z.dtype, device=z.device)
    r, ti = rows(z), ids(t, z)
    with torch.cuda.device(dev):
        _check("vws_logprobs_bwd", L.vws_logprobs_bwd(ctypes.byref(r), ctypes.byref(ti), ignore_index, _ptr(stats),
                                                      _ptr(g), gs, _ptr(dz), _stream(dev)))
    return dz


def logprobs_topk_fwd(z, ids, ignore_index=-100, split_hint=0):
    """(logp fp32 [N..., K], stats fp32 [N, 2]) for K ids per row -- vws_logprobs_topk_fwd."""
    dev = _device(z, ids)
    L = lib()
    ti = ids_k(ids, z)
    n = _n_rows(z)
    logp = torch.empty(tuple(z.shape[:-1]) + (ti.K,), dtype=torch.float32, device=z.device)
    stats = torch.empty((n, 2), dtype=torch.float32, device=z.device)
    ws, nb = _workspace(OP_LOGPROBS, z, split_hint)
    r = rows(z)
    with torch.cuda.device(dev):
        _check("vws_logprobs_topk_fwd", L.vws_logprobs_topk_fwd(ctypes.byref(r), ctypes.byref(ti), ignore_index,
                                                                _ptr(logp), _ptr(stats), _ptr(ws), nb, split_hint,
                                                                _stream(dev)))
    return logp, stats


def logprobs_topk_bwd(z, ids, stats, g, ignore_index=-100):
    """dz [shape of z, contiguous, dtype of z] of sum g * logp over the K slots -- vws_logprobs_topk_bwd."""
    dev = _device(z, ids, stats, g)
    L = lib()
    ti = ids_k(ids, z)
    n = _n_rows(z)
    if g.dtype != torch.float32:
        g = g.float()
    if g.numel() == 1 or all(st == 0 for st in g.stride()):
        gs_r, gs_k = 0, 0
    else:
        g = g.reshape(n, ti.K)
        gs_r, gs_k = g.stride(0), g.stride(1)
    dz = torch.empty(z.shape, dtype=z.dtype, device=z.device)
    r = rows(z)
    with torch.cuda.device(dev):
        _check("vws_logprobs_topk_bwd", L.vws_logprobs_topk_bwd(ctypes.byref(r), ctypes.byref(ti), ignore_index,
                                                                _ptr(stats), _ptr(g), gs_r, gs_k, _ptr(dz),
                                                                _stream(dev)))
    return dz


def entropy_fwd(z, split_hint=0):
    """(H fp32 [N...], stats fp32 [N, 2]) -- vws_entropy_fwd."""
    dev = _device(z)
    L = lib()
    H, stats = _outputs(z, 2)
    ws, nb = _workspace(OP_ENTROPY, z, split_hint)
    r = rows(z)
    with torch.cuda.device(dev):
        _check("vws_entropy_fwd", L.vws_entropy_fwd(ctypes.byref(r), _ptr(H), _ptr(stats), _ptr(ws), nb, split_hint,
                                                    _stream(dev)))
    return H, stats


def entropy_bwd(z, stats, H, g):
    """dz -- vws_entropy_bwd."""
    dev = _device(z, stats, H, g)
    L = lib()
    g, gs = _g_arg(g, z)
    dz = torch.empty(z.shape, dtype=z.dtype, device=z.device)
    r = rows(z)
    with torch.cuda.device(dev):
        _check("vws_entropy_bwd", L.vws_entropy_bwd(ctypes.byref(r), _ptr(stats), _ptr(H), _ptr(g), gs, _ptr(dz),
                                                    _stream(dev)))
    return dz


def kl_fwd(a, b, split_hint=0):
    """(KL(A||B) fp32 [N...], stats fp32 [N, 4]) -- vws_kl_fwd."""
    dev = _device(a, b)
    L = lib()
    kl, stats = _outputs(a, 4)
    ws, nb = _workspace(OP_KL, a, split_hint)
    ra, rb = rows(a), rows(b)
    with torch.cuda.device(dev):
        _check("vws_kl_fwd", L.vws_kl_fwd(ctypes.byref(ra), ctypes.byref(rb), _ptr(kl), _ptr(stats), _ptr(ws), nb,
                                          split_hint, _stream(dev)))
    return kl, stats


def kl_fwd_noalloc(a, b, split_hint=0):
    """(KL(A||B) fp32 [N...], stats fp32 [N, 4]) -- vws_kl_fwd_noalloc: the same results as
    kl_fwd, with the split's partial states in the library's static per-GPU buffer (the
    outputs are still allocated here, by torch)."""
    dev = _device(a, b)
    L = lib()
    kl, stats = _outputs(a, 4)
    ra, rb = rows(a), rows(b)
    with torch.cuda.device(dev):
        _check("vws_kl_fwd_noalloc", L.vws_kl_fwd_noalloc(ctypes.byref(ra), ctypes.byref(rb), _ptr(kl), _ptr(stats),
                                                          split_hint, _stream(dev)))
    return kl, stats


def kl_bwd(a, b, stats, kl, g, need_a=True, need_b=True):
    """(da or None, db or None) -- vws_kl_bwd."""
    dev = _device(a, b, stats, kl, g)
    L = lib()
    g, gs = _g_arg(g, a)
    da = torch.empty(a.shape, dtype=a.dtype, device=a.device) if need_a else None
    db = torch.empty(b.shape, dtype=b.dtype, device=b.device) if need_b else None
    ra, rb = rows(a), rows(b)
    with torch.cuda.device(dev):
        _check("vws_kl_bwd", L.vws_kl_bwd(ctypes.byref(ra), ctypes.byref(rb), _ptr(stats), _ptr(kl), _ptr(g), gs,
                                          _ptr(da), _ptr(db), _stream(dev)))
    return da, db


def jsd_fwd(s, t, beta=0.5, split_hint=0):
    """(JSD fp32 [N...], stats fp32 [N, 6]) of student s and teacher t -- vws_jsd_fwd."""
    dev = _device(s, t)
    L = lib()
    out, stats = _outputs(s, 6)
    ws, nb = _workspace(OP_JSD, s, split_hint)
    rs, rt = rows(s), rows(t)
    with torch.cuda.device(dev):
        _check("vws_jsd_fwd", L.vws_jsd_fwd(ctypes.byref(rs), ctypes.byref(rt), float(beta), _ptr(out), _ptr(stats),
                                            _ptr(ws), nb, split_hint, _stream(dev)))
    return out, stats


def jsd_bwd(s, t, beta, stats, out, g, need_s=True, need_t=True):
    """(ds or None, dt or None) -- vws_jsd_bwd."""
    dev = _device(s, t, stats, out, g)
    L = lib()
    g, gs = _g_arg(g, s)
    ds = torch.empty(s.shape, dtype=s.dtype, device=s.device) if need_s else None
    dt = torch.empty(t.shape, dtype=t.dtype, device=t.device) if need_t else None
    rs, rt = rows(s), rows(t)
    with torch.cuda.device(dev):
        _check("vws_jsd_bwd", L.vws_jsd_bwd(ctypes.byref(rs), ctypes.byref(rt), float(beta), _ptr(stats), _ptr(out),
                                            _ptr(g), gs, _ptr(ds), _ptr(dt), _stream(dev)))
    return ds, dt


# ------------------------------------------------------------- fused linear-logp

def _lin_check(h, W, t):
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("h and W must be bfloat16")
    if h.dim() != 2 or W.dim() != 2 or h.shape[1] != W.shape[1]:
        raise ValueError("h must be [N, H] and W [V, H]")
    if h.stride(1) != 1 or W.stride(1) != 1:
        raise ValueError("h and W need a contiguous last dimension")
    if t.dtype != torch.int64 or t.dim() != 1 or t.shape[0] != h.shape[0] or t.stride(0) != 1:
        raise ValueError("targets must be a contiguous int64 [N] tensor")


def linear_workspace_bytes(pass_, n, hidden, v, split_hint=0):
    r = lib().vws_linear_workspace_bytes(pass_, n, hidden, v, split_hint)
    if r == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace query")
    return r


def linear_logp_fwd(h, W, t, ignore_index=-100, split_hint=0):
    """(logp fp32 [N], stats fp32 [N, 2]) of the target under logits h W^T -- vws_linear_logp_fwd.
    split_hint: 0 automatic vocabulary chunking, k >= 1 k chunks, SPLIT_INVARIANT fixed
    1024-column chunks (batch invariant)."""
    dev = _device(h, W, t)
    L = lib()
    _lin_check(h, W, t)
    n, hidden = h.shape
    v = W.shape[0]
    logp = torch.empty(n, dtype=torch.float32, device=h.device)
    stats = torch.empty((n, 2), dtype=torch.float32, device=h.device)
    nb = linear_workspace_bytes(0, n, hidden, v, split_hint)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=h.device)
    with torch.cuda.device(dev):
        _check("vws_linear_logp_fwd", L.vws_linear_logp_fwd(h.data_ptr(), h.stride(0), W.data_ptr(), W.stride(0),
                                                            VWS_BF16, n, hidden, v, t.data_ptr(), ignore_index,
                                                            _ptr(logp), _ptr(stats), _ptr(ws), nb, split_hint,
                                                            _stream(dev)))
    return logp, stats


def linear_logp_bwd(h, W, t, stats, g, ignore_index=-100, need_h=True, need_w=True, split_hint=0, ws=None):
    """(dh bf16 [N, H] or None, dW bf16 [V, H] or None) -- vws_linear_logp_bwd.
    split_hint: 0 vocabulary chunks of 8192 columns, k >= 1 k chunks. ws: optional uint8 device
    tensor of at least linear_workspace_bytes(1, ...) bytes to use as the workspace (after the
    call it holds the last chunk's dz pair; allocated here when None)."""
    dev = _device(h, W, t, stats, g, ws)
    L = lib()
    _lin_check(h, W, t)
    n, hidden = h.shape
    v = W.shape[0]
    g, gs = _g_arg(g, h)
    dh = torch.empty((n, hidden), dtype=torch.bfloat16, device=h.device) if need_h else None
    dW = torch.empty((v, hidden), dtype=torch.bfloat16, device=h.device) if need_w else None
    nb = linear_workspace_bytes(1, n, hidden, v, split_hint)
    if ws is None:
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=h.device)
    elif ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < nb:
        raise ValueError("workspace must be a contiguous uint8 tensor of at least %d bytes" % nb)
    with torch.cuda.device(dev):
        _check("vws_linear_logp_bwd", L.vws_linear_logp_bwd(h.data_ptr(), h.stride(0), W.data_ptr(), W.stride(0),
                                                            VWS_BF16, n, hidden, v, t.data_ptr(), ignore_index,
                                                            _ptr(stats), _ptr(g), gs, _ptr(dh), _ptr(dW), _ptr(ws),
                                                            ws.numel(), split_hint, _stream(dev)))
    return dh, dW
