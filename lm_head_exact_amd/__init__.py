"""lm_head_exact_amd: exact Gumbel-Max sampling fused into the LM-head matmul
on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libflashsample.so`` (hand-written HIP
kernels, declared in ``include/flashsample.h``); the functions exported here
only marshal torch tensors into that library.  The library is loaded on first
use and a missing build raises instead of falling back to anything else.
"""
_BINDING_NAMES = ("sample", "sample_partial", "merge", "sample_partial_lse", "merge_lse", "sample_unfused", "workspace_bytes",
                  "unfused_workspace_bytes", "library_path", "debug_noise", "debug_gumbel",
                  "num_configs", "config_name", "profile_enable", "profile_read", "force_config", "selected_config",
                  "FlashSampleError", "alloc_workspace", "online_bounds", "sample_online",
                  "online_workspace_bytes", "pack_weights", "sample_packed",
                  "packed_weights_bytes", "device_info", "sample_packed_noalloc",
                  "sample_groups_lse", "groups_workspace_bytes")
__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(".binding", __name__)
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
