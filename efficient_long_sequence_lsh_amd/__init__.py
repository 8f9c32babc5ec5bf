"""Shared-QK LSH self-attention forward pass for AMD MI355X (gfx950).

The hot path (hash -> stable sort -> chunked attention -> round combine and
un-sort) runs in hand-written HIP kernels behind a C ABI (``include/reformer_lsh.h``);
this package is a thin ctypes binding over that shared library plus seeded
synthetic workloads.  Loading the library is deferred to the first call, and a
missing library raises instead of falling back to anything else.
"""
from .workloads import WORKLOADS, Workload, make_inputs  # noqa: F401

__all__ = ["WORKLOADS", "Workload", "make_inputs", "native"]


def __getattr__(name):
    if name == "native":
        from . import _native
        return _native
    raise AttributeError(name)
