"""lm_head_exact_amd: exact Gumbel-Max sampling fused into the LM-head matmul
on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libflashsample.so`` (hand-written HIP
kernels, declared in ``include/flashsample.h``); the functions exported here
only marshal torch tensors into that library.  The library is loaded on first
use and a missing build raises instead of falling back to anything else.
"""
__all__ = ["sample", "sample_partial", "merge", "sample_unfused", "workspace_bytes",
           "unfused_workspace_bytes", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
