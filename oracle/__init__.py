"""CPU oracle for exact Gumbel-Max sampling fused into the LM-head matmul.

TEST INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its binding) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only loads
the library and marshals NumPy arrays.  bf16 tensors travel as their raw
16-bit patterns (``numpy.uint16``).

Method (FlashSampling pages -- wiki summary, "Key claims" and "Method"; arXiv
abstract): score s = z / T + g with z = h . W_v and g standard Gumbel noise,
then one argmax per row over the whole vocabulary; a temperature that is not
positive means greedy (s = z).  The noise for (seed, step, row, global id gv)
is word gv mod 4 of Philox-4x32-10 at counter (gv / 4, row, step_lo,
step_hi) and key (seed_lo, seed_hi), mapped to u = (x + 1/2) 2^-32 (all 32
bits of the word) and g = -log(-log u).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_noise_bits.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint32, ctypes.c_uint32]
        lib.oracle_noise_bits.restype = ctypes.c_uint32
        lib.oracle_uniform.argtypes = [ctypes.c_uint32]
        lib.oracle_uniform.restype = ctypes.c_double
        lib.oracle_gumbel.argtypes = [ctypes.c_uint32]
        lib.oracle_gumbel.restype = ctypes.c_float
        lib.oracle_logit.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        lib.oracle_logit.restype = ctypes.c_float
        lib.oracle_logits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        lib.oracle_logits.restype = None
        lib.oracle_score.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        lib.oracle_score.restype = ctypes.c_float
        lib.oracle_sample.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
        lib.oracle_sample.restype = None
        lib.oracle_sample_logits.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_uint64, ctypes.c_int32,
                                             ctypes.c_uint64, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_sample_logits.restype = None
        lib.oracle_merge.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_merge.restype = None
        lib.oracle_noise_bits_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                                ctypes.c_uint32, ctypes.c_uint32,
                                                ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_noise_bits_range.restype = None
        for name in ("oracle_uniform_array", "oracle_gumbel_array"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
            fn.restype = None
        vp, i32, u32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
        lib.oracle_group_gumbel.argtypes = [u64, u64, u32, u32]
        lib.oracle_group_gumbel.restype = ctypes.c_float
        lib.oracle_sample_lse.argtypes = [vp, vp, i32, i32, i32, vp, u64, u64, vp, i32,
                                          vp, vp, vp, vp]
        lib.oracle_sample_lse.restype = None
        lib.oracle_merge_lse.argtypes = [vp, vp, vp, i32, i32, vp, u64, u64, vp, vp, vp, vp]
        lib.oracle_merge_lse.restype = None
        lib.oracle_lse_logits.argtypes = [vp, i32, vp, i32, vp]
        lib.oracle_lse_logits.restype = None
        lib.oracle_gumbel_max.argtypes = []
        lib.oracle_gumbel_max.restype = ctypes.c_double
        lib.oracle_max_row_norm.argtypes = [vp, i32, i32]
        lib.oracle_max_row_norm.restype = ctypes.c_double
        lib.oracle_sample_online.argtypes = [vp, vp, i32, i32, vp, i32, vp, u64, u64, vp, i32,
                                             vp, vp, vp]
        lib.oracle_sample_online.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (n <= 0: all)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def philox4x32_10(ctr, key):
    """One Philox-4x32-10 block: 4 counter words, 2 key words -> 4 words."""
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    _load().oracle_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def noise_bits(seed, step, row, gv):
    return int(_load().oracle_noise_bits(seed, step, row, gv))


def uniform(bits):
    return float(_load().oracle_uniform(bits))


def gumbel(bits):
    return float(_load().oracle_gumbel(bits))


def noise_bits_range(seed, step, row, gv0, n):
    """Raw noise words for global ids gv0 .. gv0+n-1 of one (seed, step, row)."""
    out = np.empty(int(n), np.uint32)
    _load().oracle_noise_bits_range(int(seed), int(step), int(row), int(gv0), int(n),
                                    _ptr(out))
    return out


def uniform_array(bits):
    """u = (x + 1/2) 2^-32 per word, fp64 (exact)."""
    bits = _c(bits, np.uint32)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_uniform_array(_ptr(bits), bits.size, _ptr(out))
    return out


def gumbel_array(bits):
    bits = _c(bits, np.uint32)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_gumbel_array(_ptr(bits), bits.size, _ptr(out))
    return out


def logit(h_row, w_row):
    h_row = _c(h_row, np.uint16)
    w_row = _c(w_row, np.uint16)
    assert h_row.shape == w_row.shape and h_row.ndim == 1
    return float(_load().oracle_logit(_ptr(h_row), _ptr(w_row), h_row.shape[0]))


def logits(h, W):
    """Full fp32 logits (B x V) from bf16 bit patterns h (B x D), W (V x D)."""
    h = _c(h, np.uint16)
    W = _c(W, np.uint16)
    B, D = h.shape
    V, D2 = W.shape
    assert D == D2
    z = np.empty((B, V), dtype=np.float32)
    _load().oracle_logits(_ptr(h), _ptr(W), B, D, V, _ptr(z))
    return z


def score(z, T, seed, step, row, gv):
    return float(_load().oracle_score(z, T, seed, step, row, gv))


def sample(h, W, T, seed, step, vocab_offset=0, rows=None):
    """Sample rows of one decode step.  Returns (ids, maxval, gap) per row.

    ``rows`` lists batch positions to compute (default: all of them); the
    noise of each row is keyed on its batch position.
    """
    h = _c(h, np.uint16)
    W = _c(W, np.uint16)
    T = _c(T, np.float32)
    B, D = h.shape
    V, D2 = W.shape
    assert D == D2 and T.shape == (B,)
    if rows is None:
        r = None
        n = B
    else:
        r = _c(rows, np.int32)
        assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < B))
        n = r.size
    ids = np.empty(n, np.int32)
    val = np.empty(n, np.float32)
    gap = np.empty(n, np.float32)
    if n:
        _load().oracle_sample(_ptr(h), _ptr(W), D, V, int(vocab_offset), _ptr(T),
                              int(seed), int(step), _ptr(r), n, _ptr(ids), _ptr(val),
                              _ptr(gap))
    return ids, val, gap


def sample_logits(z, T, seed0, step, n_seeds=1, vocab_offset=0, rows=None):
    """Sample from fixed fp32 logits z (R x V) for n_seeds consecutive seeds.

    T has one entry per row of z; ``rows`` gives each row's batch position
    (default 0..R-1).  Returns (ids, maxval, gap), each n_seeds x R.
    """
    z = _c(z, np.float32)
    T = _c(T, np.float32)
    R, V = z.shape
    assert T.shape == (R,)
    r = None if rows is None else _c(rows, np.int32)
    if r is not None:
        assert r.shape == (R,)
    ids = np.empty((n_seeds, R), np.int32)
    val = np.empty((n_seeds, R), np.float32)
    gap = np.empty((n_seeds, R), np.float32)
    _load().oracle_sample_logits(_ptr(z), V, int(vocab_offset), _ptr(T), int(seed0),
                                 int(n_seeds), int(step), _ptr(r), R, _ptr(ids),
                                 _ptr(val), _ptr(gap))
    return ids, val, gap


def merge(val, ids):
    """Per-row argmax over P x B partials (largest value, then smallest id)."""
    val = _c(val, np.float32)
    ids = _c(ids, np.int32)
    assert val.shape == ids.shape and val.ndim == 2
    P, B = val.shape
    out_id = np.empty(B, np.int32)
    out_val = np.empty(B, np.float32)
    _load().oracle_merge(_ptr(val), _ptr(ids), P, B, _ptr(out_id), _ptr(out_val))
    return out_id, out_val


# ---------------------------------------------------------------------------
# Grouped (hierarchical) sampler: oracle.c, "Grouped (hierarchical) sampler".
# ---------------------------------------------------------------------------
def group_gumbel(seed, step, row, p):
    """Gumbel draw of group p for a batch row (disjoint from token noise)."""
    return float(_load().oracle_group_gumbel(int(seed), int(step), int(row), int(p)))


def sample_lse(h, W, T, seed, step, vocab_offset=0, rows=None):
    """As ``sample``, plus the log-sum-exp of each row's scaled logits over
    the slice (greedy rows: the largest logit).  Returns (ids, val, gap, lse)."""
    h = _c(h, np.uint16)
    W = _c(W, np.uint16)
    T = _c(T, np.float32)
    B, D = h.shape
    V, D2 = W.shape
    assert D == D2 and T.shape == (B,)
    r = None if rows is None else _c(rows, np.int32)
    n = B if r is None else r.size
    ids = np.empty(n, np.int32)
    val = np.empty(n, np.float32)
    gap = np.empty(n, np.float32)
    lse = np.empty(n, np.float32)
    if n:
        _load().oracle_sample_lse(_ptr(h), _ptr(W), D, V, int(vocab_offset), _ptr(T),
                                  int(seed), int(step), _ptr(r), n, _ptr(ids), _ptr(val),
                                  _ptr(gap), _ptr(lse))
    return ids, val, gap, lse


def lse_logits(z, T):
    """Log-sum-exp of fixed fp32 logits z (R x V), one per row."""
    z = _c(z, np.float32)
    T = _c(T, np.float32)
    R, V = z.shape
    assert T.shape == (R,)
    out = np.empty(R, np.float32)
    _load().oracle_lse_logits(_ptr(z), V, _ptr(T), R, _ptr(out))
    return out


def merge_lse(val, ids, lse, T, seed, step):
    """Grouped merge of P x B partials (val, ids, lse), group p in row p.
    Returns (ids, val, total_lse, key_gap) per batch row."""
    val = _c(val, np.float32)
    ids = _c(ids, np.int32)
    lse = _c(lse, np.float32)
    T = _c(T, np.float32)
    assert val.shape == ids.shape == lse.shape and val.ndim == 2
    P, B = val.shape
    assert T.shape == (B,)
    out_id = np.empty(B, np.int32)
    out_val = np.empty(B, np.float32)
    out_lse = np.empty(B, np.float32)
    out_gap = np.empty(B, np.float32)
    _load().oracle_merge_lse(_ptr(val), _ptr(ids), _ptr(lse), P, B, _ptr(T), int(seed),
                             int(step), _ptr(out_id), _ptr(out_val), _ptr(out_lse),
                             _ptr(out_gap))
    return out_id, out_val, out_lse, out_gap


# ---------------------------------------------------------------------------
# Online (chunked) sampler with early finalisation: oracle.c, "Online
# (chunked) sampler with early finalisation".
# ---------------------------------------------------------------------------
def gumbel_max():
    """Largest value of the Gumbel map (top word), -log(-log(1 - 2^-33))."""
    return float(_load().oracle_gumbel_max())


def max_row_norm(W):
    """Largest Euclidean row norm of W (bf16 bits, V x D), fp64."""
    W = _c(W, np.uint16)
    V, D = W.shape
    return float(_load().oracle_max_row_norm(_ptr(W), V, D))


def sample_online(h, W, T, seed, step, cuts, vocab_offset=0, rows=None):
    """Chunks W[cuts[c]:cuts[c+1]] in order with early finalisation per row.
    Returns (ids, val, chunks_used)."""
    h = _c(h, np.uint16)
    W = _c(W, np.uint16)
    T = _c(T, np.float32)
    cuts = _c(cuts, np.int32)
    B, D = h.shape
    V, D2 = W.shape
    assert D == D2 and T.shape == (B,)
    assert cuts[0] == 0 and cuts[-1] == V and np.all(np.diff(cuts) > 0)
    r = None if rows is None else _c(rows, np.int32)
    n = B if r is None else r.size
    ids = np.empty(n, np.int32)
    val = np.empty(n, np.float32)
    used = np.empty(n, np.int32)
    if n:
        _load().oracle_sample_online(_ptr(h), _ptr(W), D, int(vocab_offset), _ptr(cuts),
                                     cuts.size - 1, _ptr(T), int(seed), int(step), _ptr(r), n,
                                     _ptr(ids), _ptr(val), _ptr(used))
    return ids, val, used
