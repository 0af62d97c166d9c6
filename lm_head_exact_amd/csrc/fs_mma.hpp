// fs_mma.hpp -- the LM-head contraction tile on gfx950 bf16 MFMA.
//
// A wavefront computes (MR*16 vocabulary rows) x (NT*16 batch rows) of
// logits z[b][v] = sum_d h[b][d] W[v][d] with v_mfma_f32_16x16x32_bf16: W is
// the MFMA "A" operand (rows = vocabulary), h the "B" operand (columns =
// batch).  Every W element is used by one wave only, so W fragments go
// straight from global memory into registers; h, shared by all waves of a
// block, is read through L1/L2 or staged in LDS.
//
// Register layouts (wave64, 16x16x32 bf16):
//   A fragment, lane l: row (l % 16), 8 consecutive k at 8 * (l / 16)
//   B fragment, lane l: col (l % 16), the same 8 k
//   C tile,     lane l: col (l % 16), rows 4 * (l / 16) + {0,1,2,3}
// A lane loads 16 contiguous bytes of one W row per 32-wide k step and ends up
// holding four consecutive vocabulary rows of one batch row: exactly the four
// ids one Philox block covers.
//
// Main-loop policies (all with the same interface, see fused_sample_kernel):
//   StreamLoop  each wave owns MR*16 rows and the whole of D; both operands
//               from global memory, P k-steps of loads in flight.
//   KSplitLoop  the NW waves of a block share MR*16 rows and split D into NW
//               slices; partial accumulators are summed through LDS in a
//               fixed wave order.  Blocks are small and short-lived, so the
//               rows being streamed at any moment form a narrow window of W,
//               which keeps HBM row-buffer locality high (small batches).
//   LdsLoop     each wave owns MR*16 rows; h is staged through LDS in
//               KC-wide chunks (double-buffered, XOR-swizzled 16-byte pieces)
//               and shared by the block's waves (large batches).
//   DmaLoop     as LdsLoop, but h reaches LDS by direct buffer->LDS loads in
//               an S-deep ring, with explicit load-count waits so that the W
//               stream keeps its lead across chunk barriers (large batches).
// Rows outside [0, V) and batch rows >= B read clamped (valid) addresses; their
// results are discarded by the epilogue, so operands need no masking except for the
// k >= D tail of the stream loop.  W loads may use the non-temporal hint (NTL):
// each W byte is read exactly once, so it should not displace h in the caches.
#pragma once

#include "fs_device.hpp"

namespace fs {

// Rows outside [0, V) (the ragged end, and the rows before 0 of a grid that
// is shifted to align global ids) read a valid row; their results are masked.
__device__ __forceinline__ int clamp_row(int r, int32_t V) { return min(max(r, 0), V - 1); }

template <bool NTL = false>
__device__ __forceinline__ bf16x8 load_frag(const __bf16* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, NTL ? __builtin_nontemporal_load(q) : *q);
}

// Packed W (fragment order).  The vocabulary grid's 16-row groups are stored
// one after another, each k-step by k-step as the 64 lanes' 16-byte A-fragment
// pieces: element ((g * (D / 32) + s) * 64 + l) * 8 + j holds
// W[16 g + (l % 16) - shift][32 s + 8 (l / 16) + j], zero for rows outside
// [0, V), with shift = vocab_offset mod 4 (the grid's alignment of global ids).
// A fragment load then reads 1 KB contiguous and a group's k-steps follow one
// another in memory, so each wave streams its groups front to back instead of
// taking 64 bytes from each of 16 rows 8 KB apart (HBM page locality).
constexpr int kPackedStep = kWave * 8;  // elements from one k-step of a group to the next

// The lane's piece of k-step 0 of group g.
__device__ __forceinline__ const __bf16* packed_frag(const __bf16* Wp, int g, int32_t D, int lane) {
  return Wp + (static_cast<size_t>(g) * (D / 32) * kWave + lane) * 8;
}

__device__ __forceinline__ bf16x8 zero_frag() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int MR, int NT>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MR][NT]) {
  static_for<MR>([&](auto m) FS_INLINE {
    static_for<NT>([&](auto n) FS_INLINE { acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f}; });
  });
}

// acc[m][n] += A[m] * B[n] for every (m, n) of the wave's block.
template <int MR, int NT>
__device__ __forceinline__ void mma_step(const bf16x8 (&a)[MR], const bf16x8 (&b)[NT],
                                         f32x4 (&acc)[MR][NT]) {
  static_for<MR>([&](auto m) FS_INLINE {
    static_for<NT>([&](auto n) FS_INLINE { acc[m][n] = mfma16(a[m], b[n], acc[m][n]); });
  });
}

// Pointers to the wave's A rows (clamped to V-1) and B rows (clamped to B-1),
// each already offset to the lane's 8-element k piece and to k = kbeg.
template <int MR, int NT>
struct FragPtrs {
  const __bf16* a[MR];
  const __bf16* b[NT];
  __device__ __forceinline__ FragPtrs(const __bf16* W, const __bf16* h, int32_t B, int32_t D,
                                      int32_t V, int32_t row0, int32_t col0, int32_t kbeg) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    static_for<MR>([&](auto m) FS_INLINE {
      a[m] = W + static_cast<size_t>(clamp_row(row0 + m * 16 + li, V)) * D + kbeg + 8 * kb;
    });
    static_for<NT>([&](auto n) FS_INLINE {
      b[n] = h + static_cast<size_t>(min(col0 + n * 16 + li, B - 1)) * D + kbeg + 8 * kb;
    });
  }
  template <bool NTL>
  __device__ __forceinline__ void load(int t, bf16x8 (&af)[MR], bf16x8 (&bf)[NT]) const {
    static_for<MR>([&](auto m) FS_INLINE { af[m] = load_frag<NTL>(a[m] + t * 32); });
    static_for<NT>([&](auto n) FS_INLINE { bf[n] = load_frag<false>(b[n] + t * 32); });
  }
};

// k-steps [0, ksteps) of one wave, P steps of loads in flight.  ksteps % P
// steps at the end run unpipelined.
template <int MR, int NT, int P, bool NTL>
__device__ __forceinline__ void pipelined_ksteps(const FragPtrs<MR, NT>& ptr, int ksteps,
                                                 f32x4 (&acc)[MR][NT]) {
  const int kmain = ksteps - ksteps % P;
  bf16x8 a[P][MR], b[P][NT];
  if (kmain > 0) {
    static_for<P>([&](auto p) FS_INLINE { ptr.template load<NTL>(p, a[p], b[p]); });
    for (int t0 = P; t0 < kmain; t0 += P) {
      static_for<P>([&](auto p) FS_INLINE {
        mma_step(a[p], b[p], acc);
        ptr.template load<NTL>(t0 + p, a[p], b[p]);
      });
    }
    static_for<P>([&](auto p) FS_INLINE { mma_step(a[p], b[p], acc); });
  }
  for (int t = kmain; t < ksteps; ++t) {
    bf16x8 af[MR], bfr[NT];
    ptr.template load<NTL>(t, af, bfr);
    mma_step(af, bfr, acc);
  }
}

// ---------------------------------------------------------------------------
// StreamLoop
// ---------------------------------------------------------------------------
template <int MR_, int NT_, int NW_, int P, bool NTL>
struct StreamLoop {
  static constexpr int MR = MR_, NT = NT_, NW = NW_;
  // the epilogue's per-row temperatures are loaded after the main loop
  static constexpr bool kEarlyTemperature = false;
  static constexpr int kRowsPerBlock = MR * 16 * NW;
  static constexpr size_t kSmemBytes = 0;
  static constexpr int kWavesPerSimd = 1;  // occupancy hint: none
  static bool supports(int32_t /*D*/) { return true; }
  static constexpr size_t kMaxHBytes = ~size_t{0};
  static constexpr int kBlockCols = NT * 16;
  __device__ __forceinline__ static int row0(int block, int wave) { return (block * NW + wave) * MR * 16; }
  __device__ __forceinline__ static int col_off(int /*wave*/) { return 0; }
  __device__ __forceinline__ static bool owns(int /*wave*/, int /*m*/, int /*n*/) { return true; }

  __device__ __forceinline__ static void run(const __bf16* __restrict__ W, const __bf16* __restrict__ h,
                             int32_t B, int32_t D, int32_t V, int32_t row0, int32_t col0,
                             f32x4 (&acc)[MR][NT], void* /*smem*/) {
    const FragPtrs<MR, NT> ptr(W, h, B, D, V, row0, col0, 0);
    zero_acc(acc);
    const int ksteps = D >> 5;
    pipelined_ksteps<MR, NT, P, NTL>(ptr, ksteps, acc);
    if (D & 31) {  // D % 8 == 0: a lane's 8 k are all inside or all outside
      const int kb = (threadIdx.x & (kWave - 1)) >> 4;
      const bool kin = ksteps * 32 + 8 * kb < D;
      bf16x8 af[MR], bfr[NT];
      static_for<MR>([&](auto m) FS_INLINE { af[m] = kin ? load_frag(ptr.a[m] + ksteps * 32) : zero_frag(); });
      static_for<NT>([&](auto n) FS_INLINE { bfr[n] = kin ? load_frag(ptr.b[n] + ksteps * 32) : zero_frag(); });
      mma_step(af, bfr, acc);
    }
  }
};

// ---------------------------------------------------------------------------
// KSplitLoop: requires D % (32 * NW) == 0.
// ---------------------------------------------------------------------------
template <int MR_, int NT_, int NW_, int P, bool NTL>
struct KSplitLoop {
  static constexpr int MR = MR_, NT = NT_, NW = NW_;
  // the epilogue's per-row temperatures are loaded after the main loop
  static constexpr bool kEarlyTemperature = false;
  static constexpr int kRowsPerBlock = MR * 16;
  static constexpr size_t kSmemBytes = static_cast<size_t>(NW) * MR * NT * kWave * sizeof(f32x4);
  static constexpr int kWavesPerSimd = 1;
  static bool supports(int32_t D) { return D % (32 * NW) == 0; }
  static constexpr size_t kMaxHBytes = ~size_t{0};
  static constexpr int kBlockCols = NT * 16;
  __device__ __forceinline__ static int row0(int block, int /*wave*/) { return block * MR * 16; }
  __device__ __forceinline__ static int col_off(int /*wave*/) { return 0; }
  // Tile (m, n) is finished (summed) by one wave; the others skip its epilogue.
  __device__ __forceinline__ static bool owns(int wave, int m, int n) { return (m * NT + n) % NW == wave; }

  __device__ __forceinline__ static void run(const __bf16* __restrict__ W, const __bf16* __restrict__ h,
                             int32_t B, int32_t D, int32_t V, int32_t row0, int32_t col0,
                             f32x4 (&acc)[MR][NT], void* smem) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int kw = D / NW;
    const FragPtrs<MR, NT> ptr(W, h, B, D, V, row0, col0, wave * kw);
    zero_acc(acc);
    pipelined_ksteps<MR, NT, P, NTL>(ptr, kw >> 5, acc);

    f32x4* red = static_cast<f32x4*>(smem);
    static_for<MR>([&](auto m) FS_INLINE {
      static_for<NT>([&](auto n) FS_INLINE { red[((wave * MR + m) * NT + n) * kWave + lane] = acc[m][n]; });
    });
    __syncthreads();
    static_for<MR>([&](auto m) FS_INLINE {
      static_for<NT>([&](auto n) FS_INLINE {
        if (owns(wave, m, n)) {
          f32x4 s = red[((0 * MR + m) * NT + n) * kWave + lane];
          for (int w = 1; w < NW; ++w) s += red[((w * MR + m) * NT + n) * kWave + lane];
          acc[m][n] = s;
        }
      });
    });
  }
};

// ---------------------------------------------------------------------------
// LdsLoop: h staged through LDS in KC-wide chunks; W fragments stream through
// a ring of P k-steps that runs ahead of the MFMAs across chunk boundaries.
// Requires D % (KC * U) == 0 with U the chunk unroll below.
// ---------------------------------------------------------------------------
template <int MR_, int NT_, int NW_, int KC, int P, bool NTL, int WB_ = 1, int BR = 0>
struct LdsLoop {
  static constexpr int MR = MR_, NT = NT_, NW = NW_;
  // the epilogue's per-row temperatures are loaded after the main loop
  static constexpr bool kEarlyTemperature = false;
  // The block's waves form WR row groups x WB batch groups: with WB > 1 each
  // W row group is computed by WB waves against different batch rows, which
  // halves (WB = 2) the LDS bytes read per MFMA for the same accumulators.
  static constexpr int WB = WB_, WR = NW / WB;
  static_assert(NW % WB == 0, "waves must tile the block");
  static constexpr int kRowsPerBlock = MR * 16 * WR;
  static constexpr int kBlockCols = NT * 16 * WB;
  static constexpr int N = kBlockCols;      // batch rows per block (staged in LDS)
  static constexpr int KS = KC / 32;        // MFMA k-steps per chunk
  static constexpr int CPR = KC / 8;        // 16-byte pieces per staged row
  static constexpr int THREADS = NW * kWave;
  static constexpr int LOADS = N * CPR / THREADS;  // staging loads per thread
  static constexpr int STAGE = N * KC;      // bf16 elements per buffer
  static constexpr size_t kSmemBytes = 2 * STAGE * sizeof(__bf16);
  // Chunks per unrolled loop body: even (LDS buffer parity) and a whole
  // number of ring turns (ring slots are then compile-time constants).
  static constexpr int unroll() {
    int u = 2;
    while ((u * KS) % P != 0) u += 2;
    return u;
  }
  static constexpr int U = unroll();
  // Two waves per SIMD whenever the accumulators (MR*NT*4 registers) leave
  // room: one wave's epilogue and barriers then overlap the other's MFMAs.
  static constexpr int kWavesPerSimd = MR * NT * 4 <= 128 ? 2 : 1;
  static_assert(N * CPR % THREADS == 0, "staging must divide evenly");
  static_assert((CPR & (CPR - 1)) == 0, "KC/8 must be a power of two");
  static bool supports(int32_t D) { return D % (KC * U) == 0; }
  static constexpr size_t kMaxHBytes = ~size_t{0};
  __device__ __forceinline__ static int row0(int block, int wave) {
    return (block * WR + wave / WB) * MR * 16;
  }
  __device__ __forceinline__ static int col_off(int wave) { return (wave % WB) * NT * 16; }
  __device__ __forceinline__ static bool owns(int /*wave*/, int /*m*/, int /*n*/) { return true; }

  // Piece j of staged row n lives at slot j ^ (n mod CPR): the 16 rows a
  // B-fragment read touches at one k land in distinct bank groups.
  __device__ __forceinline__ static int smem_off(int n, int j) {
    return n * KC + ((j ^ (n & (CPR - 1))) << 3);
  }

  __device__ __forceinline__ static void stage_load(const __bf16* __restrict__ h, int32_t B,
                                                    int32_t D, int32_t col0, int c,
                                                    u32x4 (&reg)[LOADS]) {
    static_for<LOADS>([&](auto i) FS_INLINE {
      const int idx = threadIdx.x + i * THREADS;
      const int n = idx / CPR, j = idx % CPR;
      const int b = min(col0 + n, B - 1);
      reg[i] = *reinterpret_cast<const u32x4*>(h + static_cast<size_t>(b) * D + c * KC + j * 8);
    });
  }

  __device__ __forceinline__ static void stage_store(__bf16* buf, const u32x4 (&reg)[LOADS]) {
    static_for<LOADS>([&](auto i) FS_INLINE {
      const int idx = threadIdx.x + i * THREADS;
      const int n = idx / CPR, j = idx % CPR;
      *reinterpret_cast<u32x4*>(buf + smem_off(n, j)) = reg[i];
    });
  }

  // B fragment of batch tile n at k step s of the chunk in `buf`.
  __device__ __forceinline__ static bf16x8 bfrag(const __bf16* buf, int s, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    const int c0 = col_off(threadIdx.x >> 6);
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(buf + smem_off(c0 + n * 16 + li, s * 4 + kb)));
  }

  // One 32-wide k step (s-th of the chunk in `buf`) against all NT batch tiles.
  __device__ __forceinline__ static void kstep(const __bf16* buf, int s, const bf16x8 (&a)[MR],
                                               f32x4 (&acc)[MR][NT]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    const int c0 = col_off(threadIdx.x >> 6);
    static_for<NT>([&](auto n) FS_INLINE {
      const bf16x8 bf = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(buf + smem_off(c0 + n * 16 + li, s * 4 + kb)));
      static_for<MR>([&](auto m) FS_INLINE { acc[m][n] = mfma16(a[m], bf, acc[m][n]); });
    });
  }

  // PACKED: W is in fragment order (packed_frag), row0 is the wave's first
  // grid row (a multiple of 16, not shifted) and V the number of groups.
  static constexpr bool kPackedW = true;
  template <bool PACKED = false>
  __device__ __forceinline__ static void run(const __bf16* __restrict__ W,
                                             const __bf16* __restrict__ h, int32_t B, int32_t D,
                                             int32_t V, int32_t row0, int32_t col0,
                                             f32x4 (&acc)[MR][NT], void* smem) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    __bf16* hs = static_cast<__bf16*>(smem);
    constexpr int kStep = PACKED ? kPackedStep : 32;  // elements between k-steps
    const __bf16* arow[MR];
    static_for<MR>([&](auto m) FS_INLINE {
      if constexpr (PACKED)
        arow[m] = packed_frag(W, min(row0 / 16 + static_cast<int>(m), V - 1), D, lane);
      else
        arow[m] = W + static_cast<size_t>(clamp_row(row0 + m * 16 + li, V)) * D + 8 * kb;
    });
    zero_acc(acc);

    // nch is a multiple of U (see supports), so the unrolled body below has
    // no branch: every load is issued unconditionally, indices past the end
    // are clamped (their data is never used), and the in-order vmcnt
    // accounting lets each k step wait only for its own fragments.
    const int nch = D / KC, nks = D / 32;
    u32x4 hreg[LOADS];
    bf16x8 ring[P][MR];
    stage_load(h, B, D, col0, 0, hreg);
    static_for<P>([&](auto p) FS_INLINE {
      const int q = min(static_cast<int>(p), nks - 1);
      static_for<MR>([&](auto m) FS_INLINE { ring[p][m] = load_frag<NTL>(arow[m] + q * kStep); });
    });
    stage_store(hs, hreg);
    __syncthreads();

    // chunk c uses LDS buffer c % 2; k step q uses ring slot q % P
    for (int c0 = 0; c0 < nch; c0 += U) {
      static_for<U>([&](auto u) FS_INLINE {
        const int c = c0 + u;
        stage_load(h, B, D, col0, min(c + 1, nch - 1), hreg);
        const __bf16* buf = hs + (u & 1) * STAGE;
        if constexpr (BR == 0) {
          static_for<KS>([&](auto s) FS_INLINE {
            constexpr int slot = (decltype(u)::value * KS + decltype(s)::value) % P;
            kstep(buf, s, ring[slot], acc);
            const int q = min(c * KS + s + P, nks - 1);
            static_for<MR>([&](auto m) FS_INLINE {
              ring[slot][m] = load_frag<NTL>(arow[m] + q * kStep);
            });
          });
        } else {
          // B fragments of the chunk's (k step, batch tile) sequence are read
          // BR ahead of their MFMAs; scheduling fences keep the reads early so
          // LDS latency overlaps MFMA work instead of stalling it.
          constexpr int T = KS * NT;
          bf16x8 bq[BR];
          static_for<BR>([&](auto t) FS_INLINE { bq[t] = bfrag(buf, t / NT, t % NT); });
          static_for<T>([&](auto tc) FS_INLINE {
            constexpr int t = decltype(tc)::value, s = t / NT, n = t % NT;
            constexpr int slot = (decltype(u)::value * KS + s) % P;
            const bf16x8 cur = bq[t % BR];
            if constexpr (t + BR < T) bq[t % BR] = bfrag(buf, (t + BR) / NT, (t + BR) % NT);
            static_for<MR>([&](auto m) FS_INLINE {
              acc[m][n] = mfma16(ring[slot][m], cur, acc[m][n]);
            });
            if constexpr (n == NT - 1) {  // k step s done: refill its W slot
              const int q = min(c * KS + s + P, nks - 1);
              static_for<MR>([&](auto m) FS_INLINE {
                ring[slot][m] = load_frag<NTL>(arow[m] + q * kStep);
              });
            }
            __builtin_amdgcn_sched_barrier(0);
          });
        }
        stage_store(hs + ((u + 1) & 1) * STAGE, hreg);  // after the last chunk: unused
        __syncthreads();
      });
    }
  }
};

// ---------------------------------------------------------------------------
// DmaLoop: the block's waves form WR = NW/WB row groups x WB batch groups;
// each wave computes MR*16 vocabulary rows against NT*16 batch rows (with
// WB = 2 the two waves of a row group read the same W rows, the second
// mostly from cache, and each reads only its half of the staged batch rows
// from LDS: half the LDS bytes per MFMA).  h is staged into LDS by direct
// global->LDS loads (no register round trip, no LDS store instructions) in a
// ring of S KC-wide chunks issued S-1 chunks ahead; W fragments stream into a
// ring of P k-steps held in registers.  Loads complete in issue order, so each
// chunk's wait names the exact number of younger loads it may leave in flight:
// the W stream keeps its P-step lead across chunk boundaries.
// Requires D % (KC * U) == 0.
// ---------------------------------------------------------------------------
template <int MR_, int NT_, int NW_, int KC, int P, int S, int BR, int G = 1, bool ROT = false,
          int WB_ = 1, bool NTL = false>
struct DmaLoop {
  static constexpr int MR = MR_, NT = NT_, NW = NW_;
  static constexpr int WB = WB_, WR = NW / WB;
  static_assert(NW % WB == 0, "waves must tile the block");
  // the epilogue's per-row temperatures are loaded after the main loop
  // (loaded before it they would hold registers the loop needs)
  static constexpr bool kEarlyTemperature = false;
  static constexpr int kRowsPerBlock = MR * 16 * WR;
  static constexpr int kBlockCols = NT * 16 * WB;
  static constexpr int KS = KC / 32;                 // MFMA k-steps per chunk
  static constexpr int CPR = KC / 8;                 // 16-byte pieces per staged row
  static constexpr int STAGE = kBlockCols * KC;      // bf16 elements per ring slot
  static constexpr int IPW = kBlockCols * CPR / (NW * kWave);  // direct loads per wave per chunk
  static_assert(kBlockCols * CPR % (NW * kWave) == 0, "staging must divide evenly");
  static_assert((CPR & (CPR - 1)) == 0, "KC/8 must be a power of two");
  static_assert(S >= 2 && BR >= 1 && BR <= KS * NT, "ring shapes");
  static constexpr size_t kSmemBytes = static_cast<size_t>(S) * STAGE * sizeof(__bf16);
  static constexpr int kWavesPerSimd = (NW + 3) / 4;
  // W slots are refilled in bursts of G consecutive k-steps, so that the
  // 64*G bytes a row contributes to one burst reach the memory controller
  // together and share DRAM page openings.
  static_assert(P % G == 0 && P >= G, "the W ring is refilled in whole bursts");
  // chunks per unrolled body: a whole number of W ring turns
  static constexpr int unroll() {
    int u = 1;
    while ((u * KS) % P != 0) ++u;
    return u;
  }
  static constexpr int U = unroll();
  // A lower bound on the loads a wave issues after chunk c+1's staging loads
  // and before the end of chunk c: S-2 younger staging groups plus the W
  // bursts completed in the S-1 chunks between (the ring prefill, P k-steps,
  // stands in for them in the first chunks).
  static constexpr int kWindowW = G * (((S - 1) * KS) / G);
  static constexpr int kYounger = (S - 2) * IPW + MR * (P < kWindowW ? P : kWindowW);
  static_assert(kYounger <= 63, "vmcnt holds at most 63");
  static bool supports(int32_t D) { return D % (KC * U) == 0; }
  static constexpr size_t kMaxHBytes = 0x7FFFFFFF;  // buffer offsets are 32-bit
  // raw buffer resource word 3 for gfx9-family parts (untyped 32-bit data)
  static constexpr int kBufferFlags = 0x00020000;
  __device__ __forceinline__ static int row0(int block, int wave) {
    return (block * WR + wave / WB) * MR * 16;
  }
  __device__ __forceinline__ static int col_off(int wave) { return (wave % WB) * NT * 16; }
  __device__ __forceinline__ static bool owns(int /*wave*/, int /*m*/, int /*n*/) { return true; }

  // Piece j of staged row n lives at slot j ^ (n mod CPR).
  __device__ __forceinline__ static int smem_off(int n, int j) {
    return n * KC + ((j ^ (n & (CPR - 1))) << 3);
  }

  // Chunk c of the block's h rows into ring slot `buf`.  Load i of wave w
  // fills the 64 consecutive 16-byte slots starting at (w*IPW + i)*64, lane
  // l the slot p = that + l: staged row n = p / CPR holding k-piece
  // (p % CPR) ^ (n % CPR), the inverse of smem_off's swizzle.  The loads are
  // buffer loads (32-bit byte offsets into h, so 2*B*D < 2^31): unlike the
  // global form they are not counted as possible LDS accesses of unknown
  // order, which would force every B-fragment read to drain the LDS queue.
  __device__ __forceinline__ static void stage(const __bf16* __restrict__ h, int32_t B, int32_t D,
                                               int32_t col0, int c, __bf16* buf) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(h), 0, B * D * 2, kBufferFlags);
    static_for<IPW>([&](auto i) FS_INLINE {
      const int base = (wave * IPW + i) * kWave;
      const int p = base + lane;
      const int n = p / CPR, j = (p % CPR) ^ (n & (CPR - 1));
      const int b = min(col0 + n, B - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, buf + base * 8, 16,
                                               (b * D + c * KC + j * 8) * 2, 0, 0, 0);
    });
  }

  // s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
  template <int N>
  __device__ __forceinline__ static void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  }

  // Workgroup barrier without the release fence of __syncthreads: that fence
  // would wait for every outstanding load, W fragments included, because
  // staging loads write LDS.  Each wave has already waited for its own staging
  // loads of the next chunk (wait_vm), and every B-fragment read of the
  // current chunk has been consumed by an MFMA, so LDS is consistent here;
  // the empty asm with a memory clobber and the scheduling fences keep the
  // compiler from moving LDS accesses across the barrier.
  __device__ __forceinline__ static void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ static bf16x8 bfrag(const __bf16* buf, int s, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    const int c0 = col_off(threadIdx.x >> 6);
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(buf + smem_off(c0 + n * 16 + li, s * 4 + kb)));
  }

  // PACKED: W is in fragment order (packed_frag), row0 is the wave's first
  // grid row (a multiple of 16, not shifted) and V the number of groups.
  static constexpr bool kPackedW = true;
  template <bool PACKED = false>
  __device__ __forceinline__ static void run(const __bf16* __restrict__ W,
                                             const __bf16* __restrict__ h, int32_t B, int32_t D,
                                             int32_t V, int32_t row0, int32_t col0,
                                             f32x4 (&acc)[MR][NT], void* smem) {
    const int lane = threadIdx.x & (kWave - 1);
    const int li = lane & 15, kb = lane >> 4;
    __bf16* hs = static_cast<__bf16*>(smem);
    constexpr int kStep = PACKED ? kPackedStep : 32;  // elements between k-steps
    const __bf16* arow[MR];
    static_for<MR>([&](auto m) FS_INLINE {
      if constexpr (PACKED)
        arow[m] = packed_frag(W, min(row0 / 16 + static_cast<int>(m), V - 1), D, lane);
      else
        arow[m] = W + static_cast<size_t>(clamp_row(row0 + m * 16 + li, V)) * D + 8 * kb;
    });
    zero_acc(acc);

    // Every load is issued unconditionally (indices past the end are clamped
    // and their data never used), so the per-chunk load counts are constants.
    const int nch = D / KC, nks = D / 32;
    // ROT: each block runs its chunks in a rotated order, starting at a
    // block-dependent chunk, so that the blocks' concurrent W reads fall on
    // different offsets of their rows (the rows are a power of two apart).
    const int r0 = ROT ? static_cast<int>((blockIdx.x * 37u) % static_cast<unsigned>(nch)) : 0;
    auto rc = [&](int c) FS_INLINE { const int x = c + r0; return x >= nch ? x - nch : x; };
    auto rq = [&](int q) FS_INLINE { const int x = q + r0 * KS; return x >= nks ? x - nks : x; };
    // The waits below count loads by issue order, so the prologue's groups are
    // fenced: staging of chunks 0 .. S-2 in order, then the W ring.
    static_for<S - 1>([&](auto s) FS_INLINE {
      stage(h, B, D, col0, rc(min(static_cast<int>(s), nch - 1)), hs + s * STAGE);
      __builtin_amdgcn_sched_barrier(0);
    });
    bf16x8 ring[P][MR];
    static_for<P>([&](auto p) FS_INLINE {
      const int q = rq(min(static_cast<int>(p), nks - 1));
      static_for<MR>([&](auto m) FS_INLINE { ring[p][m] = load_frag<NTL>(arow[m] + q * kStep); });
    });
    __builtin_amdgcn_sched_barrier(0);
    // Chunk 0 staged.  The count leaves only chunks 1 .. S-2 in flight and
    // not the W ring: the ring loads read memory the compiler knows to be
    // unchanging, so it may still move them below this wait and the barrier
    // (it does when the loop below could run zero times); counted here they
    // would then let chunk 0 be read before it lands.  With the ring issued
    // first, the wait also covers the ring, whose first slot the first MFMA
    // needs at once anyway.
    wait_vm<(S - 2) * IPW>();
    barrier();

    // nch >= U (supports), so the body runs at least once: no branch around
    // the loop that would invite the compiler to sink the prologue into it
    int slot_c = 0;  // ring slot of chunk c
    int c0 = 0;
    do {
      static_for<U>([&](auto u) FS_INLINE {
        const int c = c0 + u;
        const int slot_n = slot_c == 0 ? S - 1 : slot_c - 1;  // slot of chunk c + S - 1
        stage(h, B, D, col0, rc(min(c + S - 1, nch - 1)), hs + slot_n * STAGE);
        __builtin_amdgcn_sched_barrier(0);
        const __bf16* buf = hs + slot_c * STAGE;
        constexpr int T = KS * NT;
        bf16x8 bq[BR];
        static_for<BR>([&](auto t) FS_INLINE { bq[t] = bfrag(buf, t / NT, t % NT); });
        static_for<T>([&](auto tc) FS_INLINE {
          constexpr int t = decltype(tc)::value, s = t / NT, n = t % NT;
          constexpr int slot = (decltype(u)::value * KS + s) % P;
          const bf16x8 cur = bq[t % BR];
          if constexpr (t + BR < T) bq[t % BR] = bfrag(buf, (t + BR) / NT, (t + BR) % NT);
          static_for<MR>([&](auto m) FS_INLINE { acc[m][n] = mfma16(ring[slot][m], cur, acc[m][n]); });
          // k-step g = c*KS + s done; at the end of each G-step burst refill
          // the burst's slots with the k-steps P ahead
          constexpr int g = decltype(u)::value * KS + s;  // g mod (U*KS)
          if constexpr (n == NT - 1 && (g + 1) % G == 0) {
            static_for<G>([&](auto j) FS_INLINE {
              constexpr int sl = (g + 1 - G + decltype(j)::value) % P;
              const int q = rq(min(c * KS + s + 1 - G + decltype(j)::value + P, nks - 1));
              static_for<MR>([&](auto m) FS_INLINE { ring[sl][m] = load_frag<NTL>(arow[m] + q * kStep); });
            });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        wait_vm<kYounger>();  // chunk c + 1 staged (this wave's share)
        barrier();            // ... and every wave's; slot c is free again
        slot_c = slot_c == S - 1 ? 0 : slot_c + 1;
      });
      c0 += U;
    } while (c0 < nch);
    wait_vm<0>();  // the trailing (clamped) staging loads land before LDS is reused
  }
};

}  // namespace fs
