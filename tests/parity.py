"""Parity rules between the HIP sampler and the CPU oracle.

Bar (from the problem statement of this library):
  * the winning perturbed score agrees within 1e-3 absolute on every row;
  * the sampled id is bit-exact on every row whose oracle top-two gap
    exceeds 2e-3;
  * on a row with a smaller gap several ids are within rounding of the
    maximum, so the GPU's id is accepted when its own oracle score is within
    2e-3 of the oracle's maximum.
Only the oracle produces expected values; the GPU result is never fed back
into it.
"""
import numpy as np
import torch

import oracle
from lm_head_exact_amd import workloads as wl

VAL_TOL = 1e-3
GAP_TOL = 2e-3


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def check_rows(hb, Wb, T, seed, step, vocab_offset, ids, val, rows=None, label=""):
    """Compare GPU outputs ids/val (length B, host arrays) with the oracle on
    the listed rows (default: all).  hb, Wb: bf16 bit patterns (numpy)."""
    B = hb.shape[0]
    rows = np.arange(B, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    o_ids, o_val, o_gap = oracle.sample(hb, Wb, T, seed, step, vocab_offset, rows)
    g_ids, g_val = ids[rows], val[rows]
    err = np.abs(g_val.astype(np.float64) - o_val.astype(np.float64))
    bad_val = np.nonzero(~(err <= VAL_TOL))[0]
    assert bad_val.size == 0, (
        f"{label}: maxval off on rows {rows[bad_val][:8]}: gpu {g_val[bad_val][:8]} "
        f"oracle {o_val[bad_val][:8]}")
    exact = o_gap > GAP_TOL
    mism = np.nonzero(exact & (g_ids != o_ids))[0]
    assert mism.size == 0, (
        f"{label}: ids differ on rows {rows[mism][:8]}: gpu {g_ids[mism][:8]} "
        f"oracle {o_ids[mism][:8]} gap {o_gap[mism][:8]}")
    for i in np.nonzero(~exact & (g_ids != o_ids))[0]:
        b, gv = int(rows[i]), int(g_ids[i])
        v = gv - vocab_offset
        assert 0 <= v < Wb.shape[0], f"{label}: row {b} id {gv} outside the vocabulary"
        z = oracle.logit(hb[b], Wb[v])
        s = oracle.score(z, float(T[b]), seed, step, b, gv)
        assert o_val[i] - s <= GAP_TOL, (
            f"{label}: near-tie row {b}: gpu id {gv} scores {s}, oracle max {o_val[i]}")
    return dict(rows=len(rows), max_val_err=float(err.max()) if err.size else 0.0,
                near_ties=int((~exact).sum()))


def inputs_host_and_device(wlk, B, device="cuda", gen_device=None):
    """(h, W, T) on the device plus their host bit patterns for the oracle."""
    gen_device = gen_device or ("cpu" if wlk.w_bytes() < (64 << 20) else device)
    h = wl.make_h(wlk, B, gen_device).to(device)
    W = wl.make_w(wlk, gen_device).to(device)
    T = wl.make_temperature(wlk, B, device)
    return h, W, T, wl.bf16_bits(h), wl.bf16_bits(W), to_host(T)


def sample_rows(B, k=8, seed=0):
    """Rows checked at full size: first, last and a seeded spread."""
    if B <= k:
        return np.arange(B, dtype=np.int32)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, B - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, B - 1], mid])).astype(np.int32)
