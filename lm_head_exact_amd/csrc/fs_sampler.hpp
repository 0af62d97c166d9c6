// fs_sampler.hpp -- the fused LM-head + Gumbel-Max sampler kernels and the
// host-side launchers of their configurations.
//
// FlashSampling (wiki summary, "Method"; arXiv abstract): compute each
// vocabulary tile's logits on chip, scale by 1/T, add per-element Gumbel
// noise, keep one (max, argmax) pair per row and per tile, and finish with a
// small reduction over tiles.  Because the argmax of logits plus noise
// decomposes over any partition of the vocabulary ("Key claims"), the result
// equals one global argmax over the full noise field.  With LSE the kernels
// also emit each tile's log-sum-exp of the scaled logits, for the grouped
// (hierarchical) sampler.
//
// Grid: x = vocabulary blocks of Loop::kRowsPerBlock rows, y = batch blocks of
// NT * 16 rows (an XcdPaired loop uses a 1-D grid of the same blocks; see
// block_tile below).  The main loop (fs_mma.hpp) is a policy that leaves each
// wave with MFMA accumulators for MR * 16 vocabulary rows x NT * 16 batch
// rows; the epilogue runs in registers on those accumulators and the block
// writes one (max, argmax) partial per batch row to part_[val|idx][b][block].
//
// The configurations are instantiated in several translation units
// (fs_configs_*.hip) so that they compile in parallel.
#pragma once

#include <atomic>
#include <type_traits>

#include "fs_internal.hpp"
#include "fs_mma.hpp"

namespace fs {

// A main loop wrapped in XcdPaired runs on a 1-D grid in which the batch
// blocks of one vocabulary tile are 8 block ids apart.  Blocks are dealt to
// the 8 XCDs round robin, so those blocks run on one XCD at nearly the same
// time, and all but the first find the tile's W rows in that XCD's L2: a
// narrower batch tile (more MFMAs per B fragment read from LDS) without
// reading W from HBM once per batch block.
template <class L>
struct XcdPaired : L {
  static constexpr bool kXcdPaired = true;
};
// Main loops that can read W in fragment order (packed_frag) declare kPackedW.
template <class L, class = void>
struct reads_packed_w : std::false_type {};
template <class L>
struct reads_packed_w<L, std::void_t<decltype(L::kPackedW)>> : std::bool_constant<L::kPackedW> {};

template <class L, class = void>
struct is_xcd_paired : std::false_type {};
template <class L>
struct is_xcd_paired<L, std::void_t<decltype(L::kXcdPaired)>>
    : std::bool_constant<L::kXcdPaired> {};

constexpr int kXcds = 8;

// Batch blocks per call, and grid blocks per launch.
template <class Loop>
__host__ __device__ inline int batch_blocks(int32_t B) {
  return (B + Loop::kBlockCols - 1) / Loop::kBlockCols;
}

// (vocabulary tile, batch block) of this block; tile >= S marks a padding
// block of the paired grid.
template <class Loop>
__device__ __forceinline__ void block_tile(const SampleArgs& a, int& tile, int& bblock) {
  if constexpr (is_xcd_paired<Loop>::value) {
    const int per_group = kXcds * batch_blocks<Loop>(a.B);
    const int g = blockIdx.x / per_group, w = blockIdx.x % per_group;
    tile = g * kXcds + w % kXcds;
    bblock = w / kXcds;
  } else {
    tile = blockIdx.x;
    bblock = blockIdx.y;
  }
}

template <class Loop, bool LSE, bool PACKED = false>
__global__ __launch_bounds__(Loop::NW * kWave)
__attribute__((amdgpu_waves_per_eu(Loop::kWavesPerSimd))) void fused_sample_kernel(SampleArgs a) {
  constexpr int MR = Loop::MR, NT = Loop::NT, NW = Loop::NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  int tile, bblock;
  block_tile<Loop>(a, tile, bblock);
  if (tile >= a.S) return;  // padding block of a paired grid (block-uniform)
  if (a.live != nullptr && *a.live == 0) return;  // nothing left to sample (uniform)
  // The block's vocabulary group in a grouped launch: its first row, its row
  // count and its first block (the whole of W otherwise).  The table is read
  // with constant indices only (a kernel-argument array indexed at run time
  // could be copied to scratch memory); the scan is block-uniform.
  int g_row0 = 0, g_rows = a.V, g_tile0 = 0;
  if (a.n_groups > 0) {
#pragma unroll
    for (int k = 0; k < kMaxGroups; ++k) {
      if (k < a.n_groups && a.grp_tiles[k] <= tile) {
        g_row0 = a.grp_rows[k];
        g_rows = a.grp_rows[k + 1] - a.grp_rows[k];
        g_tile0 = a.grp_tiles[k];
      }
    }
  }
  // The group's block grid starts (vocab_offset + g_row0) mod 4 rows before its
  // first row, so that every lane's four consecutive rows begin at a global id
  // divisible by 4; fragment-order W is packed on the grid of the whole of W,
  // shifted by vocab_offset mod 4.
  const int shift = (a.vocab_offset + g_row0) & 3;
  const int pack_shift = a.vocab_offset & 3;
  const int row0 = g_row0 + Loop::row0(tile - g_tile0, wave) - shift;
  const int block_col0 = bblock * Loop::kBlockCols;

  const int col0 = block_col0 + Loop::col_off(wave);  // this wave's first batch row
  // The temperatures of the wave's batch rows are loaded all at once, before
  // the main loop where the loop leaves registers for them, else right after
  // it: loaded next to their uses, each batch tile would wait one full memory
  // latency of a busy HBM.
  float temp[NT];
  auto load_temperatures = [&]() FS_INLINE {
    static_for<NT>([&](auto n) FS_INLINE {
      temp[n] = a.temperature[min(col0 + static_cast<int>(n) * 16 + li, a.B - 1)];
    });
  };
  if constexpr (Loop::kEarlyTemperature) load_temperatures();

  f32x4 acc[MR][NT];
  if constexpr (PACKED)  // fragment-order W: groups of the unshifted grid
    Loop::template run<true>(a.W, a.h, a.B, a.D, (a.V + pack_shift + 15) / 16, row0 + pack_shift,
                             block_col0, acc, dyn_smem);
  else
    Loop::run(a.W, a.h, a.B, a.D, a.V, row0, block_col0, acc, dyn_smem);
  if constexpr (!Loop::kEarlyTemperature) load_temperatures();

  // ---- epilogue: scale, perturb, running (max, argmax) per batch row ----
  // Lane (li, kb) holds batch row col0 + 16n + li and vocabulary rows
  // row0 + 16m + 4kb + r, r = 0..3: one Philox block (global ids from a
  // multiple of 4); rows outside the block's group never win.
  // With a log-sum-exp output (grouped sampler) the same pass also keeps a
  // running log-sum-exp of the scaled logits per batch row.
  const Philox philox(a.seed);
  ArgMax best[NT];
  LseAcc lacc[NT];
  {
    static_for<NT>([&](auto n) FS_INLINE {
      best[n].init();
      if (LSE) lacc[n].init();
      // rows b >= B run on a clamped temperature; their results are not written
      const int b = col0 + n * 16 + li;
      const float T = temp[n];
      const bool greedy = row_is_greedy(T);
      const float inv_t = row_inv_temperature(T);
      static_for<MR>([&](auto m) FS_INLINE {
        if (Loop::owns(wave, m, n)) {
          const int v0 = row0 + m * 16 + 4 * kb;  // vocab_offset + v0 is a multiple of 4
          push_four<LSE>(best[n], acc[m][n], v0 - g_row0, g_rows,
                                 static_cast<uint32_t>(a.vocab_offset + v0),
                                 static_cast<uint32_t>(b), a.step, greedy, inv_t, philox,
                                 &lacc[n]);
        }
      });
    });
    // lanes l, l^16, l^32, l^48 hold the same batch row
    static_for<NT>([&](auto n) FS_INLINE {
      best[n].xor_reduce(16);
      best[n].xor_reduce(32);
      if (LSE) {
        lacc[n].xor_reduce(16);
        lacc[n].xor_reduce(32);
      }
    });
  }

  __shared__ float s_val[NW][NT * 16];
  __shared__ int32_t s_idx[NW][NT * 16];
  if (kb == 0) {
    static_for<NT>([&](auto n) FS_INLINE {
      s_val[wave][n * 16 + li] = best[n].v;
      s_idx[wave][n * 16 + li] = best[n].i;
    });
  }
  __syncthreads();
  // block column c is covered by the waves w with col_off(w) == c - c % (NT*16)
  for (int c = threadIdx.x; c < Loop::kBlockCols; c += NW * kWave) {
    const int b = block_col0 + c;
    if (b >= a.B) break;
    ArgMax m;
    m.init();
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (Loop::col_off(w) == c - c % (NT * 16)) m.push(s_val[w][c % (NT * 16)], s_idx[w][c % (NT * 16)]);
    const size_t o = static_cast<size_t>(b) * a.S + tile;
    a.part_val[o] = m.v;
    a.part_idx[o] = m.i;
  }
  if constexpr (LSE) {  // the same two arrays carry the (m, s) pairs
    __syncthreads();
    if (kb == 0) {
      static_for<NT>([&](auto n) FS_INLINE {
        s_val[wave][n * 16 + li] = lacc[n].m;
        s_idx[wave][n * 16 + li] = __float_as_int(lacc[n].s);
      });
    }
    __syncthreads();
    for (int c = threadIdx.x; c < Loop::kBlockCols; c += NW * kWave) {
      const int b = block_col0 + c;
      if (b >= a.B) break;
      LseAcc l;
      l.init();
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (Loop::col_off(w) == c - c % (NT * 16))
          l.merge(s_val[w][c % (NT * 16)], __int_as_float(s_idx[w][c % (NT * 16)]));
      a.part_lse[static_cast<size_t>(b) * a.S + tile] = l.value(row_is_greedy(a.temperature[b]));
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent K-split sampler for small batches (NT * 16 batch rows).
//
// Block = NW waves, one or two per SIMD, launched once per CU slot.  Wave w
// owns the D-slice [w*KS*32, (w+1)*KS*32) and keeps h for that slice in
// registers for the whole kernel, so h is read from memory once per block.
// Blocks sweep the 16-row vocabulary groups g = block, block + G, ...: the
// groups being streamed at any moment form a narrow moving window of W,
// which keeps HBM row-buffer locality high.  W fragments stream through a
// P-deep register ring that runs ahead across group boundaries.  After each
// group the NW partial accumulators are summed through LDS (two buffers,
// fixed wave order) by one owner wave per batch tile, which runs the
// epilogue; ownership rotates over the waves.  The running (max, argmax)
// persists across groups, so a block emits one partial per batch row.
//
// GROUPED (a grouped launch, log-sum-exps included): the 16-row groups are
// those of each vocabulary group's own grid (see SampleArgs), numbered
// group after group, so a block meets the vocabulary groups in increasing
// order.  The owner of batch tile n is fixed within a vocabulary group, so
// the group's running pair sits in one wave, which writes it when the block
// moves on: entry t of each row, t the block's first 16-row group in that
// vocabulary group.  Vocabulary group g's partials are therefore entries
// [grp_tiles[g], min(grp_tiles[g+1], grp_tiles[g] + grid size)).
// Requires D == 32 * NW * KS.
// ---------------------------------------------------------------------------
template <int NT, int NW, int KS, int P, bool LSE, bool PACKED = false, bool NTL = false,
          bool GROUPED = false>
__global__ __launch_bounds__(NW * kWave) void persist_sample_kernel(SampleArgs a) {
  static_assert(KS % P == 0, "the load ring must tile a group");
  static_assert(!GROUPED || LSE, "grouped launches carry log-sum-exps");
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  f32x4* red = reinterpret_cast<f32x4*>(dyn_smem);  // [2][NW][NT][kWave]
  if (a.live != nullptr && *a.live == 0) return;  // nothing left to sample (uniform)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  const int D = a.D;
  const int kbeg = wave * KS * 32 + 8 * kb;
  // 16-row groups over a vocabulary grid shifted as in the tiled kernel
  const int shift = a.vocab_offset & 3;
  const int ngroups = GROUPED ? a.S : (a.V + shift + 15) / 16;
  const int G = gridDim.x;
  // Grouped launch: the group table, copied once into LDS (entry k by thread
  // k) and then read at the vocabulary group of a cursor that only moves
  // forward, since a block's 16-row groups come in increasing order.
  __shared__ int32_t s_grp_rows[GROUPED ? kMaxGroups + 1 : 1];
  __shared__ int32_t s_grp_tiles[GROUPED ? kMaxGroups + 1 : 1];
  if constexpr (GROUPED) {
    const int k = static_cast<int>(threadIdx.x);
    if (k <= a.n_groups) {
      s_grp_rows[k] = a.grp_rows[k];
      s_grp_tiles[k] = a.grp_tiles[k];
    }
    __syncthreads();
  }
  // The cursor's vocabulary group: index, first row, row count, first
  // 16-row group, and the next group's first 16-row group (the table entries
  // are the same on every lane: read into scalar registers, and only when the
  // cursor moves).
  int cursor = 0, c_row0 = 0, c_rows = a.V, c_tile0 = 0, c_next = 0x7FFFFFFF;
  auto load_cursor = [&]() FS_INLINE {
    c_row0 = __builtin_amdgcn_readfirstlane(s_grp_rows[cursor]);
    c_rows = __builtin_amdgcn_readfirstlane(s_grp_rows[cursor + 1]) - c_row0;
    c_tile0 = __builtin_amdgcn_readfirstlane(s_grp_tiles[cursor]);
    c_next = cursor + 1 < a.n_groups ? __builtin_amdgcn_readfirstlane(s_grp_tiles[cursor + 1])
                                     : 0x7FFFFFFF;
  };
  if constexpr (GROUPED) load_cursor();
  // 16-row group t (non-decreasing from call to call): its first row (a row
  // of W, negative before row 0) and, in a grouped launch, its vocabulary
  // group (index, first row, row count).  t is block-uniform.
  struct Rows { int row0, grp, g_row0, g_rows; };
  auto rows_of = [&](int t) FS_INLINE {
    const int tc = min(t, ngroups - 1);
    Rows r{tc * 16 - shift, 0, 0, a.V};
    if constexpr (GROUPED) {
      while (tc >= c_next) {
        ++cursor;
        load_cursor();
      }
      r.grp = cursor;
      r.g_row0 = c_row0;
      r.g_rows = c_rows;
      r.row0 = c_row0 - ((a.vocab_offset + c_row0) & 3) + 16 * (tc - c_tile0);
    }
    return r;
  };

  bf16x8 hreg[KS][NT];
  bool bvalid[NT], greedy[NT];
  float inv_t[NT];
  static_for<NT>([&](auto n) FS_INLINE {
    const int b = n * 16 + li;
    bvalid[n] = b < a.B;
    const __bf16* hp = a.h + static_cast<size_t>(min(b, a.B - 1)) * D + kbeg;
    static_for<KS>([&](auto s) FS_INLINE { hreg[s][n] = load_frag(hp + s * 32); });
    const float T = bvalid[n] ? a.temperature[b] : 1.0f;
    greedy[n] = row_is_greedy(T);
    inv_t[n] = row_inv_temperature(T);
  });

  // PACKED: W in fragment order (packed_frag): the 16 rows from row0 are
  // packed group (row0 + shift) / 16 (vocabulary groups of a packed grouped
  // launch start at multiples of 16, so their grids are the packed one)
  constexpr int kStep = PACKED ? kPackedStep : 32;  // elements between k-steps
  auto group_ptr = [&](const Rows& r) FS_INLINE {
    if constexpr (PACKED)
      return packed_frag(a.W, (r.row0 + shift) >> 4, D, lane) + wave * KS * kPackedStep;
    else
      return a.W + static_cast<size_t>(clamp_row(r.row0 + li, a.V)) * D + kbeg;
  };
  const Philox philox(a.seed);
  ArgMax best[NT];
  LseAcc lacc[NT];  // grouped sampler only: running log-sum-exp per batch row
  static_for<NT>([&](auto n) FS_INLINE {
    best[n].init();
    if (LSE) lacc[n].init();
  });

  int g = blockIdx.x;
  Rows cur = rows_of(g), nxt = rows_of(g + G);
  const __bf16* ap = group_ptr(cur);
  const __bf16* ap_next = group_ptr(nxt);
  // grouped launch: the vocabulary group whose pairs the block holds, and
  // the entry they go to
  int open_grp = -1, open_slot = 0;
  auto flush_group = [&]() FS_INLINE {
    static_for<NT>([&](auto n) FS_INLINE {
      if ((n + open_grp) % NW == wave) {  // wave-uniform: the group's owner of tile n
        best[n].xor_reduce(16);
        best[n].xor_reduce(32);
        lacc[n].xor_reduce(16);
        lacc[n].xor_reduce(32);
        if (kb == 0 && bvalid[n]) {
          const size_t o = static_cast<size_t>(n * 16 + li) * a.S + open_slot;
          a.part_val[o] = best[n].v;
          a.part_idx[o] = best[n].i;
          a.part_lse[o] = lacc[n].value(greedy[n]);
        }
        best[n].init();
        lacc[n].init();
      }
    });
  };
  bf16x8 ring[P];
  static_for<P>([&](auto p) FS_INLINE { ring[p] = load_frag<NTL>(ap + p * kStep); });

  for (int it = 0; g < ngroups; g += G, ++it) {
    f32x4 acc[NT];
    static_for<NT>([&](auto n) FS_INLINE { acc[n] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    static_for<KS>([&](auto sc) FS_INLINE {
      constexpr int s = decltype(sc)::value;
      constexpr int slot = s % P;
      static_for<NT>([&](auto n) FS_INLINE { acc[n] = mfma16(ring[slot], hreg[s][n], acc[n]); });
      // refill with the k-step P ahead (the next group's, past the end of this one)
      if constexpr (s + P < KS)
        ring[slot] = load_frag<NTL>(ap + (s + P) * kStep);
      else
        ring[slot] = load_frag<NTL>(ap_next + (s + P - KS) * kStep);
    });
    const Rows here = cur;
    cur = nxt;
    nxt = rows_of(g + 2 * G);
    ap = ap_next;
    ap_next = group_ptr(nxt);

    const int par = it & 1;
    static_for<NT>([&](auto n) FS_INLINE {
      red[((par * NW + wave) * NT + n) * kWave + lane] = acc[n];
    });
    __syncthreads();
    if constexpr (GROUPED) {
      if (here.grp != open_grp) {  // block-uniform
        if (open_grp >= 0) flush_group();
        open_grp = here.grp;
        open_slot = g;
      }
    }
    // the owner of tile n rotates with the 16-row group (with the vocabulary
    // group in a grouped launch)
    const int turn = GROUPED ? here.grp : it;
    static_for<NT>([&](auto n) FS_INLINE {
      if ((n + turn) % NW == wave && bvalid[n]) {
        f32x4 z = red[((par * NW + 0) * NT + n) * kWave + lane];
        for (int w = 1; w < NW; ++w) z += red[((par * NW + w) * NT + n) * kWave + lane];
        const int b = n * 16 + li;
        const int v0 = here.row0 + 4 * kb;  // ids grow with g for each owner
        const uint32_t gv0 = static_cast<uint32_t>(a.vocab_offset + v0);
        push_four<LSE>(best[n], z, v0 - here.g_row0, here.g_rows, gv0,
                       static_cast<uint32_t>(b), a.step, greedy[n], inv_t[n], philox, &lacc[n]);
      }
    });
  }
  if constexpr (GROUPED) {
    if (open_grp >= 0) flush_group();
    return;
  }

  static_for<NT>([&](auto n) FS_INLINE {
    best[n].xor_reduce(16);
    best[n].xor_reduce(32);
    if (LSE) {
      lacc[n].xor_reduce(16);
      lacc[n].xor_reduce(32);
    }
  });
  __shared__ float s_val[NW][NT * 16];
  __shared__ int32_t s_idx[NW][NT * 16];
  if (kb == 0) {
    static_for<NT>([&](auto n) FS_INLINE {
      s_val[wave][n * 16 + li] = best[n].v;
      s_idx[wave][n * 16 + li] = best[n].i;
    });
  }
  __syncthreads();
  for (int c = threadIdx.x; c < NT * 16 && c < a.B; c += NW * kWave) {
    ArgMax m;
    m.init();
#pragma unroll
    for (int w = 0; w < NW; ++w) m.push(s_val[w][c], s_idx[w][c]);
    const size_t o = static_cast<size_t>(c) * a.S + blockIdx.x;
    a.part_val[o] = m.v;
    a.part_idx[o] = m.i;
  }
  if constexpr (LSE) {  // the same two arrays carry the (m, s) pairs
    __syncthreads();
    if (kb == 0) {
      static_for<NT>([&](auto n) FS_INLINE {
        s_val[wave][n * 16 + li] = lacc[n].m;
        s_idx[wave][n * 16 + li] = __float_as_int(lacc[n].s);
      });
    }
    __syncthreads();
    for (int c = threadIdx.x; c < NT * 16 && c < a.B; c += NW * kWave) {
      LseAcc l;
      l.init();
#pragma unroll
      for (int w = 0; w < NW; ++w) l.merge(s_val[w][c], __int_as_float(s_idx[w][c]));
      a.part_lse[static_cast<size_t>(c) * a.S + blockIdx.x] = l.value(row_is_greedy(a.temperature[c]));
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: launchers and the configuration entries built from them.
// ---------------------------------------------------------------------------

// Raises the dynamic-LDS limit of a kernel once (it may exceed the default).
template <class Kernel>
hipError_t allow_smem(Kernel kernel, size_t smem) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
}

template <class Loop>
hipError_t launch_cfg(SampleArgs& a, hipStream_t stream) {
  constexpr int rows = Loop::kRowsPerBlock;
  static_assert(rows >= kMinRowsPerBlock, "split count bound");
  if (!Loop::supports(a.D) || static_cast<size_t>(a.B) * a.D * 2 > Loop::kMaxHBytes)
    return hipErrorInvalidValue;
  constexpr size_t smem = Loop::kSmemBytes;
  if (smem > 0) {
    static const hipError_t attr = [] {
      const hipError_t e = allow_smem(&fused_sample_kernel<Loop, false>, smem);
      return e != hipSuccess ? e : allow_smem(&fused_sample_kernel<Loop, true>, smem);
    }();
    if (attr != hipSuccess) return attr;
  }
  if (a.n_groups > 0) {  // each group's blocks start at its own first row
    a.grp_tiles[0] = 0;
    for (int g = 0; g < a.n_groups; ++g) {
      const int grows = a.grp_rows[g + 1] - a.grp_rows[g];
      const int gshift = (a.vocab_offset + a.grp_rows[g]) & 3;
      a.grp_tiles[g + 1] = a.grp_tiles[g] + (grows + gshift + rows - 1) / rows;
    }
    a.S = a.grp_tiles[a.n_groups];
    a.grp_span = 0;
  } else {
    a.S = (a.V + (a.vocab_offset & 3) + rows - 1) / rows;
  }
  const int nb = batch_blocks<Loop>(a.B);
  // grid limits: x < 2^31 blocks, y <= 65535 (checked here, before launching)
  const int64_t paired_x = static_cast<int64_t>((a.S + kXcds - 1) / kXcds) * kXcds * nb;
  if (nb > 65535 || (is_xcd_paired<Loop>::value && paired_x > 0x7FFFFFFF))
    return hipErrorInvalidConfiguration;
  const dim3 grid = is_xcd_paired<Loop>::value ? dim3(static_cast<unsigned>(paired_x))
                                               : dim3(a.S, nb);
  const dim3 block(Loop::NW * kWave);
  if (a.w_packed) {
    if constexpr (reads_packed_w<Loop>::value) {
      if (smem > 0) {
        static const hipError_t attr = [] {
          const hipError_t e = allow_smem(&fused_sample_kernel<Loop, false, true>, smem);
          return e != hipSuccess ? e : allow_smem(&fused_sample_kernel<Loop, true, true>, smem);
        }();
        if (attr != hipSuccess) return attr;
      }
      if (a.part_lse == nullptr)
        fused_sample_kernel<Loop, false, true><<<grid, block, smem, stream>>>(a);
      else
        fused_sample_kernel<Loop, true, true><<<grid, block, smem, stream>>>(a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.part_lse == nullptr)
    fused_sample_kernel<Loop, false><<<grid, block, smem, stream>>>(a);
  else
    fused_sample_kernel<Loop, true><<<grid, block, smem, stream>>>(a);
  return hipGetLastError();
}

template <class Loop>
bool supports_cfg(int32_t B, int32_t D) {
  return Loop::supports(D) && static_cast<size_t>(B) * D * 2 <= Loop::kMaxHBytes;
}

// Per-device results of one kernel's occupancy query (0: not yet known).
// Each kernel keeps its own: kernels of one signature share a pointer type,
// so a cache keyed on that type would hand one kernel's answer to another.
struct OccupancyCache {
  static constexpr int kMaxDevices = 64;
  std::atomic<int> blocks[kMaxDevices];
};

// Blocks of `kernel` that fit on one CU, times the CU count of the current
// device, cached per device in `cache`.
template <class Kernel>
int resident_blocks(Kernel kernel, int threads, size_t smem, OccupancyCache& cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool cacheable = dev >= 0 && dev < OccupancyCache::kMaxDevices;
  if (cacheable) {
    const int known = cache.blocks[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, smem) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  if (cacheable) cache.blocks[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int NT, int NW, int KS, int P, bool NTL = false>
struct Persist {
  static constexpr size_t kSmemBytes = 2ull * NW * NT * kWave * sizeof(f32x4);
  static bool supports(int32_t B, int32_t D) { return B <= NT * 16 && D == 32 * NW * KS; }
  template <bool LSE, bool PACKED = false>
  static hipError_t go(SampleArgs& a, hipStream_t stream) {
    const auto kernel = persist_sample_kernel<NT, NW, KS, P, LSE, PACKED, NTL>;
    static OccupancyCache cache;  // one per kernel instantiation
    const int slots = resident_blocks(kernel, NW * kWave, kSmemBytes, cache);
    if (slots <= 0) return hipErrorInvalidDevice;
    const int ngroups = (a.V + (a.vocab_offset & 3) + 15) / 16;
    a.S = ngroups < slots ? ngroups : slots;
    kernel<<<a.S, NW * kWave, kSmemBytes, stream>>>(a);
    return hipGetLastError();
  }
  // Grouped launch: every vocabulary group on its own grid of 16-row groups
  // (its first row shifted down to a global id divisible by 4), numbered group
  // after group; a.grp_span = the grid size that bounds each group's partials.
  template <bool PACKED>
  static hipError_t go_groups(SampleArgs& a, hipStream_t stream) {
    const auto kernel = persist_sample_kernel<NT, NW, KS, P, true, PACKED, NTL, true>;
    static OccupancyCache cache;
    const int slots = resident_blocks(kernel, NW * kWave, kSmemBytes, cache);
    if (slots <= 0) return hipErrorInvalidDevice;
    a.grp_tiles[0] = 0;
    for (int g = 0; g < a.n_groups; ++g) {
      const int grows = a.grp_rows[g + 1] - a.grp_rows[g];
      const int gshift = (a.vocab_offset + a.grp_rows[g]) & 3;
      a.grp_tiles[g + 1] = a.grp_tiles[g] + (grows + gshift + 15) / 16;
    }
    a.S = a.grp_tiles[a.n_groups];
    a.grp_span = a.S < slots ? a.S : slots;
    kernel<<<a.grp_span, NW * kWave, kSmemBytes, stream>>>(a);
    return hipGetLastError();
  }
  static hipError_t launch(SampleArgs& a, hipStream_t stream) {
    if (!supports(a.B, a.D)) return hipErrorInvalidValue;
    if (a.n_groups > 0) {  // grouped launches carry log-sum-exps
      if (a.part_lse == nullptr) return hipErrorInvalidValue;
      return a.w_packed ? go_groups<true>(a, stream) : go_groups<false>(a, stream);
    }
    if (a.w_packed) return a.part_lse == nullptr ? go<false, true>(a, stream) : go<true, true>(a, stream);
    return a.part_lse == nullptr ? go<false>(a, stream) : go<true>(a, stream);
  }
};

template <class Loop>
constexpr FusedConfig make_cfg(const char* name, int order) {
  return {name, Loop::kRowsPerBlock, &launch_cfg<Loop>, &supports_cfg<Loop>, order,
          reads_packed_w<Loop>::value};
}

template <class Pol>
constexpr FusedConfig make_persist(const char* name, int order) {
  return {name, 16, &Pol::launch, &Pol::supports, order, true};
}

#define FS_STREAM(MR, NT, NW, P, NTL) \
  make_cfg<StreamLoop<MR, NT, NW, P, NTL>>("stream_mr" #MR "_nt" #NT "_nw" #NW "_p" #P "_ntl" #NTL, 0)
#define FS_KSPLIT(MR, NT, NW, P, NTL) \
  make_cfg<KSplitLoop<MR, NT, NW, P, NTL>>("ksplit_mr" #MR "_nt" #NT "_nw" #NW "_p" #P "_ntl" #NTL, NW)
#define FS_LDS(MR, NT, NW, KC, P, NTL)                                                           \
  make_cfg<LdsLoop<MR, NT, NW, KC, P, NTL>>(                                                   \
      "lds_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_ntl" #NTL, 0)
#define FS_LDSR(MR, NT, NW, KC, P, WB, BR)                                                     \
  make_cfg<LdsLoop<MR, NT, NW, KC, P, false, WB, BR>>(                                         \
      "lds_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_wb" #WB "_br" #BR, 0)
#define FS_DMA(MR, NT, NW, KC, P, S, BR)                                                      \
  make_cfg<DmaLoop<MR, NT, NW, KC, P, S, BR>>(                                               \
      "dma_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR, 0)
#define FS_DMAG(MR, NT, NW, KC, P, S, BR, G)                                                  \
  make_cfg<DmaLoop<MR, NT, NW, KC, P, S, BR, G>>(                                            \
      "dma_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G, 0)
#define FS_DMAR(MR, NT, NW, KC, P, S, BR, G)                                                  \
  make_cfg<DmaLoop<MR, NT, NW, KC, P, S, BR, G, true>>(                                      \
      "dmarot_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G, 0)
#define FS_DMAP(MR, NT, NW, KC, P, S, BR, G)                                                  \
  make_cfg<XcdPaired<DmaLoop<MR, NT, NW, KC, P, S, BR, G>>>(                                 \
      "dmapair_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G, 0)
#define FS_DMAW(MR, NT, NW, KC, P, S, BR, G, WB)                                              \
  make_cfg<DmaLoop<MR, NT, NW, KC, P, S, BR, G, false, WB>>(                                  \
      "dma_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G "_wb" #WB, 0)
#define FS_PERSISTN(NT, NW, KS, P) \
  make_persist<Persist<NT, NW, KS, P, true>>("persist_nt" #NT "_nw" #NW "_ks" #KS "_p" #P "_ntl1", 100 + NW)
#define FS_DMAN(MR, NT, NW, KC, P, S, BR, G)                                                  \
  make_cfg<DmaLoop<MR, NT, NW, KC, P, S, BR, G, false, 1, true>>(                            \
      "dma_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G "_ntl1", 0)
#define FS_DMAPN(MR, NT, NW, KC, P, S, BR, G)                                                 \
  make_cfg<XcdPaired<DmaLoop<MR, NT, NW, KC, P, S, BR, G, false, 1, true>>>(                  \
      "dmapair_mr" #MR "_nt" #NT "_nw" #NW "_kc" #KC "_p" #P "_s" #S "_br" #BR "_g" #G "_ntl1", 0)
#define FS_PERSIST(NT, NW, KS, P) \
  make_persist<Persist<NT, NW, KS, P>>("persist_nt" #NT "_nw" #NW "_ks" #KS "_p" #P, 100 + NW)

}  // namespace fs
