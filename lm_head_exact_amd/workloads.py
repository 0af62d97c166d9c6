"""Seeded synthetic LM-head decode workloads (inputs only, no sampling math).

This module draws the inputs that both the GPU path and the CPU oracle
consume: hidden states h (B x D, bf16), LM-head weights W (V x D, bf16, the
``nn.Linear.weight`` layout), per-row temperatures T (fp32) and the per-step
(seed, step) pair of the sampler.  It holds none of the method's arithmetic
and imports neither the oracle nor the HIP binding.

Shapes follow the LM heads of the models the FlashSampling paper builds on
(reference list on the mlsanity index page: Llama 3 and Qwen3) plus a
large-batch case and one tensor-parallel vocabulary shard (wiki summary,
"Method": each rank samples over its own vocabulary shard).  The pages'
end-to-end prompt workloads are not available; random weights of these
shapes stand in for them.  The kernel's run time does not depend on the
values (it has no data-dependent early exit).

Recipe (all draws from ``torch.Generator`` seeded per workload id k):
  h      N(0,1) fp32 -> optionally RMS-normalised x / sqrt(mean(x^2)+1e-6)
         -> bf16 (round to nearest even); seed 100k+1
  W      N(0, sigma^2) fp32 -> bf16; seed 100k+2
  T      constant, or U[lo, hi) per row with every 8th row (b % 8 == 7)
         set to 0 (greedy); seed 100k+3
  step i of a run uses sampler seed 1000k + i and step i.
Small tensors are drawn on the host; ``device="cuda"`` draws on the device
with torch's device generator (much faster for the 0.5-2 GB weights; the
values then differ from a host draw with the same seed, and tests that need
them on the host copy them back).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    key: int                     # workload id k: seeds derive from it
    name: str
    D: int                       # hidden size
    V: int                       # vocabulary rows held in W (a shard for TP)
    batches: Tuple[int, ...]     # batch sizes exercised
    w_std: float                 # std of the N(0, sigma^2) weights
    h_rmsnorm: bool              # RMS-normalise the hidden states
    temperature: float = 1.0     # constant temperature ...
    temp_range: Optional[Tuple[float, float]] = None  # ... or U[lo,hi) per row
    greedy_every: int = 0        # rows with b % greedy_every == greedy_every-1 get T=0
    vocab_offset: int = 0        # global id of W row 0
    global_V: int = 0            # full vocabulary (= V unless a shard)
    shards: int = 1              # tensor-parallel degree the shard belongs to
    notes: str = field(default="", compare=False)

    @property
    def h_seed(self) -> int:
        return 100 * self.key + 1

    @property
    def w_seed(self) -> int:
        return 100 * self.key + 2

    @property
    def t_seed(self) -> int:
        return 100 * self.key + 3

    def sampler_seed(self, i: int) -> Tuple[int, int]:
        """(seed, step) of decode step i: a fresh seed per step."""
        if self.key == 1:
            return (0 + i, i)
        return (1000 * self.key + i, i)

    def w_bytes(self) -> int:
        return 2 * self.V * self.D


TINY = Workload(1, "tiny", D=256, V=1000, batches=(4,), w_std=0.05, h_rmsnorm=False,
                global_V=1000, notes="parity + distribution; launch-bound")
LLAMA3_8B = Workload(2, "llama3-8b-lm-head", D=4096, V=128256,
                     batches=(1, 8, 32, 2, 4, 16, 64, 128, 256), w_std=0.02,
                     h_rmsnorm=True, global_V=128256)
QWEN3 = Workload(3, "qwen3-lm-head", D=5120, V=151936, batches=(64, 128, 256),
                 w_std=0.02, h_rmsnorm=True, temp_range=(0.3, 1.5), greedy_every=8,
                 global_V=151936)
LARGE_BATCH = Workload(4, "large-batch-lm-head", D=8192, V=128256, batches=(256, 512),
                       w_std=0.015, h_rmsnorm=False, temperature=0.7, global_V=128256)
TP8_SHARD = Workload(5, "tp8-vocab-shard", D=8192, V=16032, batches=(1, 64, 256),
                     w_std=0.015, h_rmsnorm=False, vocab_offset=3 * 16032,
                     global_V=128256, shards=8)

WORKLOADS = {w.name: w for w in (TINY, LLAMA3_8B, QWEN3, LARGE_BATCH, TP8_SHARD)}


def _gen(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def make_h(wl: Workload, B: int, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    g = _gen(wl.h_seed if seed is None else seed, device)
    x = torch.randn(B, wl.D, generator=g, device=device, dtype=torch.float32)
    if wl.h_rmsnorm:
        x = x / torch.sqrt(x.pow(2).mean(dim=1, keepdim=True) + 1e-6)
    return x.to(torch.bfloat16).contiguous()


def make_w(wl: Workload, device="cpu", V: Optional[int] = None, seed: Optional[int] = None,
           D: Optional[int] = None) -> torch.Tensor:
    V = wl.V if V is None else V
    D = wl.D if D is None else D
    g = _gen(wl.w_seed if seed is None else seed, device)
    out = torch.empty(V, D, dtype=torch.bfloat16, device=device)
    # draw in row blocks to bound the fp32 temporary
    step = max(1, (1 << 26) // max(D, 1))
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        blk = torch.randn(r1 - r0, D, generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = (blk * wl.w_std).to(torch.bfloat16)
    return out


def make_temperature(wl: Workload, B: int, device="cpu") -> torch.Tensor:
    if wl.temp_range is None:
        T = torch.full((B,), wl.temperature, dtype=torch.float32)
    else:
        lo, hi = wl.temp_range
        g = _gen(wl.t_seed, "cpu")
        T = lo + (hi - lo) * torch.rand(B, generator=g, dtype=torch.float32)
    if wl.greedy_every:
        idx = torch.arange(B)
        T[(idx % wl.greedy_every) == wl.greedy_every - 1] = 0.0
    return T.to(device)


def make_inputs(wl: Workload, B: int, device="cpu"):
    """(h, W, T) for one workload and batch size, all on ``device``."""
    return make_h(wl, B, device), make_w(wl, device), make_temperature(wl, B, device)


def make_shard_partials(B: int, P: int = 8, V_shard: int = 16032, real_slot: int = 3,
                        seed: int = 503, device="cpu"):
    """Synthetic per-shard (value, global id) partials, P x B, part-major.

    Stand-ins for the other ranks of a P-way vocabulary split: values
    12 + 1.3 N(0,1), ids uniform inside each shard's id range.  Slot
    ``real_slot`` is left at (-inf, -1) for the caller to fill.  On rows with
    b % 16 == 5 two slots carry the same large value with different ids, so
    that the smaller-id tie-break decides the row.
    """
    g = _gen(seed, "cpu")
    val = 12.0 + 1.3 * torch.randn(P, B, generator=g, dtype=torch.float32)
    off = torch.arange(P, dtype=torch.int64).unsqueeze(1) * V_shard
    idx = (off + torch.randint(0, V_shard, (P, B), generator=g)).to(torch.int32)
    tie_rows = torch.arange(B) % 16 == 5
    a, b2 = (1, 6) if P > 6 else (0, P - 1)
    if a != b2:
        val[a, tie_rows] = 40.0
        val[b2, tie_rows] = 40.0
    if 0 <= real_slot < P:
        val[real_slot] = float("-inf")
        idx[real_slot] = -1
    return val.to(device), idx.to(device)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor as a host numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def make_confident_w(wl: Workload, h: torch.Tensor, chunk_rows: int, later_std: float,
                     gain: float = 1.0, seed: Optional[int] = None,
                     device="cpu") -> torch.Tensor:
    """W (V x D) for the online sampler's early-finalisation case.

    A stand-in for a confident model whose rare tokens have small output
    embeddings: row b < B of the first chunk (rows [0, chunk_rows)) is
    parallel to batch row b of ``h``, scaled to ``gain`` times the norm a
    typical row of N(0, w_std^2) has (w_std * sqrt(D)); the other rows of the first chunk
    are N(0, w_std^2); every later row is N(0, later_std^2).
    """
    B, D = h.shape
    assert D == wl.D and B <= chunk_rows <= wl.V
    W = make_w(wl, device, seed=seed)
    g = _gen((wl.w_seed if seed is None else seed) + 7, device)
    later = wl.V - chunk_rows
    step = max(1, (1 << 26) // D)
    for r0 in range(0, later, step):
        r1 = min(later, r0 + step)
        blk = torch.randn(r1 - r0, D, generator=g, device=device, dtype=torch.float32)
        W[chunk_rows + r0:chunk_rows + r1] = (blk * later_std).to(torch.bfloat16)
    x = h.to(device=device, dtype=torch.float32)
    x = x / x.norm(dim=1, keepdim=True).clamp_min(1e-30) * (gain * wl.w_std * D ** 0.5)
    W[:B] = x.to(torch.bfloat16)
    return W
