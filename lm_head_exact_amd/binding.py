"""ctypes binding of libflashsample (C ABI in include/flashsample.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspaces are allocated with torch, and the call
goes to the library on torch's current HIP stream.  Every step of the
sampler runs in the library's kernels.  If the library is missing or fails
to load, every function raises; there is no fallback path.
"""
import ctypes
import os
import re
from typing import Optional, Tuple

import torch  # loaded first, so the library binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libflashsample.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "flashsample.h")

FS_OK, FS_ERR_INVALID_ARG, FS_ERR_UNSUPPORTED, FS_ERR_WORKSPACE, FS_ERR_HIP = range(5)


class FlashSampleError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def exported_names_from_header():
    """Names of every function the public header declares."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"FS_API\s+[\w\s\*]+?\b(fs_\w+)\s*\(", text)))


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FlashSampleError(FS_ERR_UNSUPPORTED,
                               f"{_LIB_PATH} is missing: run lm_head_exact_amd/build.py")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, u32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32,
                                  ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t)
    sample_args = [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, vp, vp, sz, vp]
    for name, args, res in [
        ("fs_workspace_bytes", [i32, i32, i32], sz),
        ("fs_unfused_workspace_bytes", [i32, i32, i32], sz),
        ("fs_sample", sample_args, ctypes.c_int),
        ("fs_sample_partial", sample_args, ctypes.c_int),
        ("fs_sample_unfused", sample_args, ctypes.c_int),
        ("fs_merge", [vp, vp, i32, i32, vp, vp, vp], ctypes.c_int),
        ("fs_sample_partial_lse", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, vp, vp, vp,
                                   sz, vp], ctypes.c_int),
        ("fs_sample_partial_lse_packed", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, vp, vp,
                                          vp, sz, vp], ctypes.c_int),
        ("fs_merge_lse", [vp, vp, vp, i32, i32, vp, u64, u64, vp, vp, vp, vp], ctypes.c_int),
        ("fs_groups_workspace_bytes", [i32, i32, i32, i32], sz),
        ("fs_sample_groups_lse", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, i32, vp, vp, vp,
                                  vp, sz, vp], ctypes.c_int),
        ("fs_sample_groups_lse_packed", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, i32, vp,
                                         vp, vp, vp, sz, vp], ctypes.c_int),
        ("fs_packed_weights_bytes", [i32, i32, i32], sz),
        ("fs_pack_weights", [vp, i32, i32, i32, vp, sz, vp], ctypes.c_int),
        ("fs_sample_packed", sample_args, ctypes.c_int),
        ("fs_sample_packed_noalloc", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, vp, vp],
         ctypes.c_int),
        ("fs_online_bounds_workspace_bytes", [i32, i32], sz),
        ("fs_online_workspace_bytes", [i32, i32, i32, i32], sz),
        ("fs_online_bounds", [vp, i32, i32, vp, i32, vp, vp, sz, vp], ctypes.c_int),
        ("fs_online_bounds_packed", [vp, i32, i32, i32, vp, i32, vp, vp, sz, vp], ctypes.c_int),
        ("fs_sample_online", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, i32, vp, vp, vp,
                              vp, vp, sz, vp], ctypes.c_int),
        ("fs_sample_online_packed", [vp, vp, i32, i32, i32, i32, vp, u64, u64, vp, i32, vp, vp,
                                     vp, vp, vp, sz, vp], ctypes.c_int),
        ("fs_debug_noise", [u64, u64, u32, u32, i64, vp, vp, vp], ctypes.c_int),
        ("fs_debug_gumbel", [vp, i64, vp, vp], ctypes.c_int),
        ("fs_device_info", [i32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)],
         ctypes.c_int),
        ("fs_num_configs", [], i32),
        ("fs_config_name", [i32], ctypes.c_char_p),
        ("fs_force_config", [i32], ctypes.c_int),
        ("fs_selected_config", [i32, i32, i32], i32),
        ("fs_selected_config_packed", [i32, i32, i32], i32),
        ("fs_selected_config_groups", [i32, i32, i32, i32], i32),
        ("fs_profile_enable", [i32], ctypes.c_int),
        ("fs_profile_read", [ctypes.POINTER(ctypes.c_int32)] + [ctypes.POINTER(ctypes.c_double)] * 3,
         ctypes.c_int),
        ("fs_status_string", [ctypes.c_int], ctypes.c_char_p),
        ("fs_last_error", [], ctypes.c_char_p),
    ]:
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _status_name(s: int) -> str:
    try:
        return lib().fs_status_string(s).decode()
    except Exception:
        return f"status {s}"


def _check(status: int):
    if status != FS_OK:
        raise FlashSampleError(status, lib().fs_last_error().decode())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _req(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(B: int, D: int, V: int) -> int:
    return int(lib().fs_workspace_bytes(B, D, V))


def unfused_workspace_bytes(B: int, D: int, V: int) -> int:
    return int(lib().fs_unfused_workspace_bytes(B, D, V))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (or better) aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _sample_common(fn_name, h, W, temperature, seed, step, vocab_offset, out_a, out_b,
                   workspace, ws_fn):
    _req(h, "h", torch.bfloat16, 2)
    _req(W, "W", torch.bfloat16, 2)
    _req(temperature, "temperature", torch.float32, 1)
    B, D = h.shape
    V, D2 = W.shape
    if D2 != D:
        raise ValueError(f"h is B x {D} but W is V x {D2}")
    if temperature.shape[0] != B:
        raise ValueError("temperature must have B entries")
    if not (h.device == W.device == temperature.device == out_a.device == out_b.device):
        raise ValueError("all tensors must be on one device")
    if workspace is None:
        workspace = alloc_workspace(ws_fn(B, D, V), h.device)
    fn = getattr(lib(), fn_name)
    _check(fn(_ptr(h), _ptr(W), B, D, V, int(vocab_offset), _ptr(temperature),
              int(seed) & (2**64 - 1), int(step) & (2**64 - 1), _ptr(out_a), _ptr(out_b),
              _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream(h.device)))


def sample(h: torch.Tensor, W: torch.Tensor, temperature: torch.Tensor, seed: int, step: int,
           vocab_offset: int = 0, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
           workspace: Optional[torch.Tensor] = None):
    """Fused LM-head + Gumbel-Max sampling: returns (ids int32[B], maxval fp32[B])."""
    B = h.shape[0]
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=h.device),
               torch.empty(B, dtype=torch.float32, device=h.device))
    ids, val = out
    _sample_common("fs_sample", h, W, temperature, seed, step, vocab_offset, ids, val,
                   workspace, workspace_bytes)
    return ids, val


def sample_partial(h, W, temperature, seed, step, vocab_offset, partial_val, partial_idx,
                   workspace=None):
    """One shard's per-row (max, global argmax) into partial_val / partial_idx (B each)."""
    _req(partial_val, "partial_val", torch.float32, 1)
    _req(partial_idx, "partial_idx", torch.int32, 1)
    _sample_common("fs_sample_partial", h, W, temperature, seed, step, vocab_offset,
                   partial_val, partial_idx, workspace, workspace_bytes)
    return partial_val, partial_idx


def sample_partial_lse(h, W, temperature, seed, step, vocab_offset, partial_val, partial_idx,
                       partial_lse, workspace=None, V=None):
    """One vocabulary group's per-row (max, global argmax) and log-sum-exp of the
    scaled logits into partial_val / partial_idx / partial_lse (B each).  W is the
    group's row-major V x D rows, or (1-D, with V given) their fragment-order
    copy from pack_weights at the same vocab_offset."""
    _req(partial_val, "partial_val", torch.float32, 1)
    _req(partial_idx, "partial_idx", torch.int32, 1)
    _req(partial_lse, "partial_lse", torch.float32, 1)
    _req(h, "h", torch.bfloat16, 2)
    packed = W.dim() == 1
    _req(W, "W", torch.bfloat16, 1 if packed else 2)
    _req(temperature, "temperature", torch.float32, 1)
    B, D = h.shape
    if packed:
        if V is None:
            raise ValueError("V is required with fragment-order W")
        need = packed_weights_bytes(V, D, vocab_offset)
        if need == 0 or W.numel() * 2 < need:
            raise ValueError(f"W_packed holds {W.numel() * 2} bytes; {need} needed")
    else:
        V, D2 = W.shape
        if D2 != D:
            raise ValueError(f"h is B x {D} but W is V x {D2}")
    if not (temperature.shape[0] == partial_val.shape[0] == partial_idx.shape[0] ==
            partial_lse.shape[0] == B):
        raise ValueError("temperature and the partials must have B entries")
    devs = {t.device for t in (h, W, temperature, partial_val, partial_idx, partial_lse)}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device")
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(B, D, V), h.device)
    fn = lib().fs_sample_partial_lse_packed if packed else lib().fs_sample_partial_lse
    _check(fn(
        _ptr(h), _ptr(W), B, D, V, int(vocab_offset), _ptr(temperature),
        int(seed) & (2**64 - 1), int(step) & (2**64 - 1), _ptr(partial_val), _ptr(partial_idx),
        _ptr(partial_lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(h.device)))
    return partial_val, partial_idx, partial_lse


def groups_workspace_bytes(B: int, D: int, V: int, n_groups: int) -> int:
    return int(lib().fs_groups_workspace_bytes(B, D, V, n_groups))


def sample_groups_lse(h: torch.Tensor, W: torch.Tensor, temperature: torch.Tensor, seed: int,
                      step: int, cuts, vocab_offset: int = 0, out=None, workspace=None,
                      V: Optional[int] = None):
    """fs_sample_groups_lse: the grouped sampler's per-group partials for the
    groups W[cuts[g]:cuts[g+1]] in one launch.  Returns (val fp32 [G][B],
    idx int32 [G][B], lse fp32 [G][B]), slot g as fs_sample_partial_lse over
    group g.  W is the row-major V x D matrix, or (1-D, V given) its
    fragment-order copy (group starts multiples of 16)."""
    packed = W.dim() == 1
    _req(h, "h", torch.bfloat16, 2)
    _req(W, "W", torch.bfloat16, 1 if packed else 2)
    _req(temperature, "temperature", torch.float32, 1)
    B, D = h.shape
    if packed:
        if V is None:
            raise ValueError("V is required with fragment-order W")
    else:
        V = W.shape[0]
        if W.shape[1] != D:
            raise ValueError("h and W must have the same D")
    c, G = _host_cuts(cuts)
    dev = h.device
    if out is None:
        out = (torch.empty(G, B, dtype=torch.float32, device=dev),
               torch.empty(G, B, dtype=torch.int32, device=dev),
               torch.empty(G, B, dtype=torch.float32, device=dev))
    pv, pi, pl = out
    if workspace is None:
        workspace = alloc_workspace(groups_workspace_bytes(B, D, V, G), dev)
    fn = lib().fs_sample_groups_lse_packed if packed else lib().fs_sample_groups_lse
    _check(fn(_ptr(h), _ptr(W), B, D, V, int(vocab_offset), _ptr(temperature),
              int(seed) & (2**64 - 1), int(step) & (2**64 - 1), c, G, _ptr(pv), _ptr(pi),
              _ptr(pl), _ptr(workspace), workspace.numel() * workspace.element_size(),
              _stream(dev)))
    return pv, pi, pl


def merge_lse(partial_val, partial_idx, partial_lse, temperature, seed, step, out=None):
    """Grouped merge of P x B group partials: returns (ids int32[B], maxval fp32[B],
    total log-sum-exp fp32[B])."""
    _req(partial_val, "partial_val", torch.float32, 2)
    _req(partial_idx, "partial_idx", torch.int32, 2)
    _req(partial_lse, "partial_lse", torch.float32, 2)
    _req(temperature, "temperature", torch.float32, 1)
    if not (partial_val.shape == partial_idx.shape == partial_lse.shape):
        raise ValueError("the partials must have the same shape")
    P, B = partial_val.shape
    if temperature.shape[0] != B:
        raise ValueError("temperature must have B entries")
    dev = partial_val.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev))
    ids, val, lse = out
    _check(lib().fs_merge_lse(_ptr(partial_val), _ptr(partial_idx), _ptr(partial_lse), P, B,
                              _ptr(temperature), int(seed) & (2**64 - 1),
                              int(step) & (2**64 - 1), _ptr(ids), _ptr(val), _ptr(lse),
                              _stream(dev)))
    return ids, val, lse


def sample_unfused(h, W, temperature, seed, step, vocab_offset=0, out=None, workspace=None):
    """Unfused baseline (logits and probabilities in device memory)."""
    B = h.shape[0]
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=h.device),
               torch.empty(B, dtype=torch.float32, device=h.device))
    ids, val = out
    _sample_common("fs_sample_unfused", h, W, temperature, seed, step, vocab_offset, ids, val,
                   workspace, unfused_workspace_bytes)
    return ids, val


def merge(partial_val: torch.Tensor, partial_idx: torch.Tensor, out=None):
    """Per-row argmax over P x B partials (largest value, then smallest id)."""
    _req(partial_val, "partial_val", torch.float32, 2)
    _req(partial_idx, "partial_idx", torch.int32, 2)
    if partial_val.shape != partial_idx.shape:
        raise ValueError("partial_val and partial_idx must have the same shape")
    P, B = partial_val.shape
    dev = partial_val.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev))
    ids, val = out
    _check(lib().fs_merge(_ptr(partial_val), _ptr(partial_idx), P, B, _ptr(ids), _ptr(val),
                          _stream(dev)))
    return ids, val


def packed_weights_bytes(V: int, D: int, vocab_offset: int = 0) -> int:
    return int(lib().fs_packed_weights_bytes(V, D, vocab_offset))


def pack_weights(W: torch.Tensor, vocab_offset: int = 0) -> torch.Tensor:
    """W (V x D bf16) in the kernels' fragment order, as a flat bf16 tensor;
    sample it with sample_packed at the same vocab_offset (mod 4)."""
    _req(W, "W", torch.bfloat16, 2)
    V, D = W.shape
    n = packed_weights_bytes(V, D, vocab_offset)
    if n == 0:
        raise FlashSampleError(FS_ERR_INVALID_ARG, f"cannot pack a {V} x {D} W (D % 32 != 0?)")
    Wp = torch.empty(n // 2, dtype=torch.bfloat16, device=W.device)
    _check(lib().fs_pack_weights(_ptr(W), V, D, int(vocab_offset), _ptr(Wp), n,
                                 _stream(W.device)))
    return Wp


def sample_packed(h: torch.Tensor, W_packed: torch.Tensor, V: int, temperature: torch.Tensor,
                  seed: int, step: int, vocab_offset: int = 0, out=None, workspace=None):
    """fs_sample on fragment-order weights (pack_weights): returns (ids, maxval),
    identical to sample() on the row-major W."""
    _req(h, "h", torch.bfloat16, 2)
    _req(W_packed, "W_packed", torch.bfloat16, 1)
    _req(temperature, "temperature", torch.float32, 1)
    B, D = h.shape
    need = packed_weights_bytes(V, D, vocab_offset)
    if need == 0 or W_packed.numel() * 2 < need:
        raise ValueError(f"W_packed holds {W_packed.numel() * 2} bytes; {need} needed")
    if temperature.shape[0] != B:
        raise ValueError("temperature must have B entries")
    dev = h.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev))
    ids, val = out
    if len({t.device for t in (h, W_packed, temperature, ids, val)}) != 1:
        raise ValueError("all tensors must be on one device")
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(B, D, V), dev)
    _check(lib().fs_sample_packed(_ptr(h), _ptr(W_packed), B, D, V, int(vocab_offset),
                                  _ptr(temperature), int(seed) & (2**64 - 1),
                                  int(step) & (2**64 - 1), _ptr(ids), _ptr(val), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev)))
    return ids, val


def sample_packed_noalloc(h: torch.Tensor, W_packed: torch.Tensor, V: int,
                          temperature: torch.Tensor, seed: int, step: int, vocab_offset: int = 0,
                          out=None):
    """fs_sample_packed_noalloc: sample_packed with the tile partials in the
    library's own per-device scratch array instead of a workspace (calls that
    overlap on one device race).  Allocates nothing when `out` is given."""
    _req(h, "h", torch.bfloat16, 2)
    _req(W_packed, "W_packed", torch.bfloat16, 1)
    _req(temperature, "temperature", torch.float32, 1)
    B, D = h.shape
    need = packed_weights_bytes(V, D, vocab_offset)
    if need == 0 or W_packed.numel() * 2 < need:
        raise ValueError(f"W_packed holds {W_packed.numel() * 2} bytes; {need} needed")
    if temperature.shape[0] != B:
        raise ValueError("temperature must have B entries")
    dev = h.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev))
    ids, val = out
    if len({t.device for t in (h, W_packed, temperature, ids, val)}) != 1:
        raise ValueError("all tensors must be on one device")
    _check(lib().fs_sample_packed_noalloc(_ptr(h), _ptr(W_packed), B, D, V, int(vocab_offset),
                                          _ptr(temperature), int(seed) & (2**64 - 1),
                                          int(step) & (2**64 - 1), _ptr(ids), _ptr(val),
                                          _stream(dev)))
    return ids, val


def _host_cuts(cuts):
    """cuts as a host int32 ctypes array (kept alive by the caller) and the chunk count."""
    c = [int(x) for x in (cuts.tolist() if hasattr(cuts, "tolist") else cuts)]
    if len(c) < 2:
        raise ValueError("cuts needs at least two entries (0 and V)")
    return (ctypes.c_int32 * len(c))(*c), len(c) - 1


def online_bounds(W: torch.Tensor, cuts, workspace: Optional[torch.Tensor] = None,
                  V: Optional[int] = None, D: Optional[int] = None, vocab_offset: int = 0):
    """later_norm (fp64 [n_chunks], device) for the online sampler over the
    chunks W[cuts[c]:cuts[c+1]]: the largest row norm after each chunk.  W is
    the row-major V x D matrix, or (1-D, with V and D given) its fragment-order
    copy from pack_weights at vocab_offset."""
    packed = W.dim() == 1
    _req(W, "W", torch.bfloat16, 1 if packed else 2)
    if packed:
        if V is None or D is None:
            raise ValueError("V and D are required with fragment-order W")
        need = packed_weights_bytes(V, D, vocab_offset)
        if need == 0 or W.numel() * 2 < need:
            raise ValueError(f"W_packed holds {W.numel() * 2} bytes; {need} needed")
    else:
        V, D = W.shape
    arr, n = _host_cuts(cuts)
    later = torch.empty(n, dtype=torch.float64, device=W.device)
    if workspace is None:
        workspace = alloc_workspace(int(lib().fs_online_bounds_workspace_bytes(V, n)), W.device)
    nbytes = workspace.numel() * workspace.element_size()
    if packed:
        _check(lib().fs_online_bounds_packed(_ptr(W), V, D, int(vocab_offset), arr, n,
                                             _ptr(later), _ptr(workspace), nbytes,
                                             _stream(W.device)))
    else:
        _check(lib().fs_online_bounds(_ptr(W), V, D, arr, n, _ptr(later), _ptr(workspace), nbytes,
                                      _stream(W.device)))
    return later


def online_workspace_bytes(B: int, D: int, V: int, n_chunks: int) -> int:
    return int(lib().fs_online_workspace_bytes(B, D, V, n_chunks))


def sample_online(h, W, temperature, seed, step, cuts, later_norm, vocab_offset=0, out=None,
                  workspace=None, V=None):
    """Online sampler with early finalisation over the chunks W[cuts[c]:cuts[c+1]]:
    returns (ids int32[B], maxval fp32[B], chunks int32[B]).  W is the row-major
    V x D matrix, or (1-D, with V given) its fragment-order copy from
    pack_weights, whose chunk starts must be multiples of 16."""
    _req(h, "h", torch.bfloat16, 2)
    packed = W.dim() == 1
    _req(W, "W", torch.bfloat16, 1 if packed else 2)
    _req(temperature, "temperature", torch.float32, 1)
    _req(later_norm, "later_norm", torch.float64, 1)
    B, D = h.shape
    if packed:
        if V is None:
            raise ValueError("V is required with fragment-order W")
        need = packed_weights_bytes(V, D, vocab_offset)
        if need == 0 or W.numel() * 2 < need:
            raise ValueError(f"W_packed holds {W.numel() * 2} bytes; {need} needed")
    else:
        V, D2 = W.shape
        if D2 != D:
            raise ValueError(f"h is B x {D} but W is V x {D2}")
    if temperature.shape[0] != B:
        raise ValueError("temperature must have B entries")
    arr, n = _host_cuts(cuts)
    if later_norm.shape[0] != n:
        raise ValueError("later_norm must have one entry per chunk")
    dev = h.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.float32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    ids, val, chunks = out
    if len({t.device for t in (h, W, temperature, later_norm, ids, val, chunks)}) != 1:
        raise ValueError("all tensors must be on one device")
    if workspace is None:
        workspace = alloc_workspace(online_workspace_bytes(B, D, V, n), dev)
    fn = lib().fs_sample_online_packed if packed else lib().fs_sample_online
    _check(fn(
        _ptr(h), _ptr(W), B, D, V, int(vocab_offset), _ptr(temperature),
        int(seed) & (2**64 - 1), int(step) & (2**64 - 1), arr, n, _ptr(later_norm), _ptr(ids),
        _ptr(val), _ptr(chunks), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev)))
    return ids, val, chunks


def debug_noise(seed: int, step: int, row: int, gv0: int, n: int, device="cuda"):
    """Device noise words (as int32 bit patterns) and Gumbel values for ids gv0..gv0+n-1."""
    bits = torch.empty(n, dtype=torch.int32, device=device)
    g = torch.empty(n, dtype=torch.float32, device=device)
    _check(lib().fs_debug_noise(int(seed), int(step), int(row), int(gv0), int(n), _ptr(bits),
                                _ptr(g), _stream(bits.device)))
    return bits, g


def debug_gumbel(bits: torch.Tensor):
    _req(bits, "bits", torch.int32, 1)
    g = torch.empty(bits.shape[0], dtype=torch.float32, device=bits.device)
    _check(lib().fs_debug_gumbel(_ptr(bits), bits.shape[0], _ptr(g), _stream(bits.device)))
    return g


def device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) the HIP runtime reports."""
    cus, clk = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().fs_device_info(int(device), ctypes.byref(cus), ctypes.byref(clk)))
    return cus.value, clk.value


def profile_enable(capacity: int):
    """Time the next `capacity` fused-kernel launches with HIP events."""
    _check(lib().fs_profile_enable(int(capacity)))


def profile_read():
    """(launches, total_ms, min_ms, max_ms) of the launches timed so far."""
    n = ctypes.c_int32()
    tot, lo, hi = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().fs_profile_read(ctypes.byref(n), ctypes.byref(tot), ctypes.byref(lo),
                                 ctypes.byref(hi)))
    return n.value, tot.value, lo.value, hi.value


def num_configs() -> int:
    return int(lib().fs_num_configs())


def config_name(i: int) -> str:
    r = lib().fs_config_name(i)
    return r.decode() if r else ""


def force_config(i: int):
    _check(lib().fs_force_config(int(i)))


def selected_config(B: int, D: int, V: int, packed: bool = False, grouped: bool = False) -> int:
    """Configuration fs_sample (packed: fs_sample_packed) would use; grouped:
    the one fs_sample_groups_lse (or its packed form) would use."""
    if grouped:
        return int(lib().fs_selected_config_groups(B, D, V, int(packed)))
    fn = lib().fs_selected_config_packed if packed else lib().fs_selected_config
    return int(fn(B, D, V))
