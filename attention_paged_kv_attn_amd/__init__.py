"""Paged-KV attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libpaged_attn.so`` (hand-written HIP
kernels: Assign -> split-K attention -> combine); ``binding`` marshals torch
tensors into its calls.  Importing this package loads nothing; the library is
loaded on first use and its absence is an error, never a fallback.
"""
__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    if name == "workloads":
        from . import workloads
        return workloads
    raise AttributeError(name)
