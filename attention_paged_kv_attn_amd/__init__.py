"""Paged-KV attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libpaged_attn.so`` (hand-written HIP
kernels: Assign -> split-K attention -> combine); ``binding`` marshals torch
tensors into its calls.  Importing this package loads nothing; the library is
loaded on first use and its absence is an error, never a fallback.
"""
import importlib

__all__ = ["binding", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
