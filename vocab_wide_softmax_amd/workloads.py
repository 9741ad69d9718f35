"""Seeded synthetic inputs for the vocab-wide softmax reductions.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle can be fed from
it. Everything is drawn on the CPU with ``torch.Generator().manual_seed(seed)``
in float32. The large normal fields (A and B's noise, or B; h and W) are drawn
in blocks of 256 leading rows, block i from its own generator seeded by
(seed, field, i), so several threads can fill them and the values do not
depend on the thread count. Everything else comes from one generator seeded
with ``seed``, in this fixed order:

    1. offset-row choice       2. mask rows and columns
    3. targets                 4. one upstream gradient g per op, in the order of ``OPS``

Offsets and masks are applied in float32, and only then are values rounded
(round-to-nearest-even) to the storage dtype. (The 64 x 1024 tiny pair is
small enough to come from the one generator: A, then B, then the rest.) The
shapes follow the pages' workloads: a 75968-column shard of a 151936-token
vocabulary (PR #8838, B70 table caption and JSD table), 8192 tokens, large
common offsets (+1e4 here; the pages test +1000) and -inf masks in B.
"""

from dataclasses import dataclass, field
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Tuple

import torch

OPS = ("logprobs", "entropy", "kl_ab", "kl_ba")
VOCAB_SHARD = 75968
OFFSET = 1.0e4


@dataclass
class Workload:
    """Host tensors of one workload.

    ``a_base``/``b_base`` are the storage tensors; ``a``/``b`` are the logical
    [N, V] views the ops read (for the strided workload, the causal-shift view
    ``base[:, :-1, :]``). ``t`` are targets with the same row decomposition,
    ``g[op]`` the fp32 upstream gradient [N] of each op.
    """

    name: str
    a_base: torch.Tensor
    b_base: torch.Tensor
    ids_base: torch.Tensor
    shifted: bool
    g: Dict[str, torch.Tensor]
    offset_rows: torch.Tensor = field(default_factory=lambda: torch.zeros(0, dtype=torch.int64))
    mask_rows: torch.Tensor = field(default_factory=lambda: torch.zeros(0, dtype=torch.int64))

    def views(self, a_base=None, b_base=None, ids_base=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        """(a, b, t) logical views over the given (default: host) bases."""
        a_base = self.a_base if a_base is None else a_base
        b_base = self.b_base if b_base is None else b_base
        ids_base = self.ids_base if ids_base is None else ids_base
        if self.shifted:
            return a_base[:, :-1, :], b_base[:, :-1, :], ids_base[:, 1:]
        return a_base, b_base, ids_base

    @property
    def a(self):
        return self.views()[0]

    @property
    def b(self):
        return self.views()[1]

    @property
    def t(self):
        return self.views()[2]


def _gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


ROW_BLOCK = 256


def _block_gen(seed: int, stream: int, i: int) -> torch.Generator:
    return _gen(((int(seed) * 1000003 + stream) * 1000003 + i) & 0x7FFFFFFFFFFF)


def _for_blocks(n: int, fill) -> None:
    """Run fill(i, r0, r1) over row blocks of ROW_BLOCK rows, on up to 16 threads."""
    nblk = (n + ROW_BLOCK - 1) // ROW_BLOCK
    spans = [(i, i * ROW_BLOCK, min(n, (i + 1) * ROW_BLOCK)) for i in range(nblk)]
    if nblk <= 1:
        for sp in spans:
            fill(*sp)
        return
    with ThreadPoolExecutor(max_workers=min(16, nblk)) as ex:
        list(ex.map(lambda sp: fill(*sp), spans))


def _normal_block(rows: int, cols: int, seed: int, stream: int, i: int, std: float) -> torch.Tensor:
    x = torch.empty(rows, cols, dtype=torch.float32)
    x.normal_(0.0, 1.0, generator=_block_gen(seed, stream, i))
    return x.mul_(std) if std != 1.0 else x


def _pick_rows(gen: torch.Generator, n: int, k: int) -> torch.Tensor:
    """k distinct rows, row 0 always included (so one row is both offset and masked)."""
    k = max(1, min(n, k))
    rest = torch.randperm(max(n - 1, 0), generator=gen)[: k - 1] + 1
    return torch.cat([torch.zeros(1, dtype=torch.int64), rest]).sort().values


def tiny_pair(seed: int = 0, n: int = 64, v: int = 1024) -> Workload:
    """Small fp32 pair: A, B i.i.d. N(0, 2^2); row 0 of both +1e4; row 1 of B has
    16 distinct columns at -inf; targets U[0, V); g ~ N(0, 1) per op."""
    gen = _gen(seed)
    a = 2.0 * torch.randn(n, v, generator=gen)
    b = 2.0 * torch.randn(n, v, generator=gen)
    offset_rows = torch.zeros(1, dtype=torch.int64)
    a[0] += OFFSET
    b[0] += OFFSET
    mask_rows = torch.ones(1, dtype=torch.int64) if n > 1 else torch.zeros(0, dtype=torch.int64)
    cols = torch.randperm(v, generator=gen)[: min(16, v)]
    if n > 1:
        b[1, cols] = float("-inf")
    t = torch.randint(0, v, (n,), generator=gen)
    g = {op: torch.randn(n, generator=gen) for op in OPS}
    return Workload("tiny fp32 pair %dx%d" % (n, v), a, b, t, False, g, offset_rows, mask_rows)


def logit_pair(n: int, v: int = VOCAB_SHARD, seed: int = 1, dtype=torch.bfloat16,
               offset_frac: float = 0.05, mask_frac: float = 0.01, mask_cols: int = 64) -> Workload:
    """A ~ N(0, 3^2), B = A + N(0, 0.5^2); a fraction of rows (row 0 included) offset
    by +1e4 in both; a fraction of rows (row 0 included) with ``mask_cols`` distinct
    B columns at -inf; targets U[0, V); g ~ N(0, 1) per op; cast to ``dtype``."""
    gen = _gen(seed)
    offset_rows = _pick_rows(gen, n, int(round(offset_frac * n)))
    mask_rows = _pick_rows(gen, n, int(round(mask_frac * n)))
    masks = {r: torch.randperm(v, generator=gen)[: min(mask_cols, v)] for r in mask_rows.tolist()}
    t = torch.randint(0, v, (n,), generator=gen)
    g = {op: torch.randn(n, generator=gen) for op in OPS}
    is_off = torch.zeros(n, dtype=torch.bool)
    is_off[offset_rows] = True
    a_out = torch.empty(n, v, dtype=dtype)
    b_out = torch.empty(n, v, dtype=dtype)

    def fill(i, r0, r1):
        a = _normal_block(r1 - r0, v, seed, 1, i, 3.0)
        b = _normal_block(r1 - r0, v, seed, 2, i, 0.5).add_(a)
        off = is_off[r0:r1]
        if bool(off.any()):
            a[off] += OFFSET
            b[off] += OFFSET
        for r, cols in masks.items():
            if r0 <= r < r1:
                b[r - r0, cols] = float("-inf")
        a_out[r0:r1] = a.to(dtype)
        b_out[r0:r1] = b.to(dtype)

    _for_blocks(n, fill)
    name = "%s logit pair %dx%d" % (str(dtype).replace("torch.", ""), n, v)
    return Workload(name, a_out, b_out, t, False, g, offset_rows, mask_rows)


def shifted_pair(batch: int = 4, seq: int = 2049, v: int = VOCAB_SHARD, seed: int = 3,
                 dtype=torch.float32) -> Workload:
    """Two independent bases [batch, seq, V] ~ N(0, 3^2), read through the view
    base[:, :-1, :] (batch*(seq-1) rows, two row strides, no copy). Token ids
    [batch, seq] U[0, V); targets are the next-token slice ids[:, 1:]."""
    gen = _gen(seed)
    ids = torch.randint(0, v, (batch, seq), generator=gen)
    n = batch * (seq - 1)
    g = {op: torch.randn(n, generator=gen) for op in OPS}
    a_out = torch.empty(batch, seq, v, dtype=dtype)
    b_out = torch.empty(batch, seq, v, dtype=dtype)
    a_flat, b_flat = a_out.view(batch * seq, v), b_out.view(batch * seq, v)

    def fill(i, r0, r1):
        a_flat[r0:r1] = _normal_block(r1 - r0, v, seed, 1, i, 3.0).to(dtype)
        b_flat[r0:r1] = _normal_block(r1 - r0, v, seed, 2, i, 3.0).to(dtype)

    _for_blocks(batch * seq, fill)
    name = "%s causal-shift pair [%d,%d,%d][:, :-1]" % (str(dtype).replace("torch.", ""), batch, seq, v)
    return Workload(name, a_out, b_out, ids, True, g)


@dataclass
class LinearWorkload:
    name: str
    h: torch.Tensor
    W: torch.Tensor
    t: torch.Tensor
    g: torch.Tensor


def linear_logp(n: int = 8192, hidden: int = 4096, v: int = 151936, seed: int = 4,
                dtype=torch.bfloat16, w_std: float = 0.02) -> LinearWorkload:
    """h ~ N(0, 1) [n, hidden]; W ~ N(0, w_std^2) [v, hidden]; targets U[0, v);
    g ~ N(0, 1) [n]; h and W cast to ``dtype``."""
    gen = _gen(seed)
    t = torch.randint(0, v, (n,), generator=gen)
    g = torch.randn(n, generator=gen)
    h = torch.empty(n, hidden, dtype=dtype)
    W = torch.empty(v, hidden, dtype=dtype)

    def fill_h(i, r0, r1):
        h[r0:r1] = _normal_block(r1 - r0, hidden, seed, 1, i, 1.0).to(dtype)

    def fill_w(i, r0, r1):
        W[r0:r1] = _normal_block(r1 - r0, hidden, seed, 2, i, w_std).to(dtype)

    _for_blocks(n, fill_h)
    _for_blocks(v, fill_w)
    return LinearWorkload("linear-logp h[%d,%d] W[%d,%d] %s" % (n, hidden, v, hidden, str(dtype).replace("torch.", "")),
                          h, W, t, g)


def workload(name: str) -> Workload:
    """The named workloads of this path.

    tiny      : 64 x 1024 fp32 pair (seed 0)
    pair1024  : 1024 x 75968 bf16 pair (seed 1) -- short N, long V
    pair8192  : 8192 x 75968 bf16 pair (seed 2) -- the pages' headline shape
    shifted   : [4, 2049, 75968] fp32 pair read as [:, :-1, :] (seed 3)
    """
    if name == "tiny":
        return tiny_pair(0)
    if name == "pair1024":
        return logit_pair(1024, seed=1)
    if name == "pair8192":
        return logit_pair(8192, seed=2)
    if name == "shifted":
        return shifted_pair(seed=3)
    raise KeyError(name)
