"""MI355X-native vocab-wide softmax reductions (logprobs, entropy, KL) over HIP.

The compute lives in ``libvws.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, declared in include/vws.h). ``vocab_wide_softmax_amd.binding`` is the
thin ctypes layer with the same entry-point names; ``vocab_wide_softmax_amd.ops``
wraps those in torch.autograd Functions. Both are imported lazily so that the
input generators in ``workloads`` stay usable where the library is not built;
the binding raises on first use when ``libvws.so`` is missing.
"""

import importlib

__all__ = ["binding", "ops", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
