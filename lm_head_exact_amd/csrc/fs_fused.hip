// fs_fused.hip -- the fused LM-head + Gumbel-Max sampler and the merge.
//
// FlashSampling (wiki summary, "Method"; arXiv abstract): compute each
// vocabulary tile's logits on chip, scale by 1/T, add per-element Gumbel
// noise, keep one (max, argmax) pair per row and per tile, and finish with a
// small reduction over tiles.  Because the argmax of logits plus noise
// decomposes over any partition of the vocabulary ("Key claims"), the result
// equals one global argmax over the full noise field.
//
// Grid: x = vocabulary blocks of Loop::kRowsPerBlock rows, y = batch blocks of
// NT * 16 rows.  The main loop (fs_mma.hpp) is a policy that leaves each
// wave with MFMA accumulators for MR * 16 vocabulary rows x NT * 16 batch
// rows; the epilogue runs in registers on those accumulators and the block
// writes one (max, argmax) partial per batch row to part_[val|idx][b][block].
#include "fs_internal.hpp"
#include "fs_mma.hpp"

namespace fs {

template <class Loop, bool ALIGN4>
__global__ __launch_bounds__(Loop::NW * kWave)
__attribute__((amdgpu_waves_per_eu(Loop::kWavesPerSimd))) void fused_sample_kernel(SampleArgs a) {
  constexpr int MR = Loop::MR, NT = Loop::NT, NW = Loop::NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  const int row0 = Loop::row0(blockIdx.x, wave);
  const int block_col0 = blockIdx.y * Loop::kBlockCols;

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
  Loop::run(a.W, a.h, a.B, a.D, a.V, row0, block_col0, acc, dyn_smem);
  if constexpr (!Loop::kEarlyTemperature) load_temperatures();

  // ---- epilogue: scale, perturb, running (max, argmax) per batch row ----
  // Lane (li, kb) holds batch row col0 + 16n + li and vocabulary rows
  // row0 + 16m + 4kb + r, r = 0..3: one Philox block when vocab_offset % 4 == 0.
  const Philox philox(a.seed);
  ArgMax best[NT];
  static_for<NT>([&](auto n) FS_INLINE {
    best[n].init();
    // rows b >= B run on a clamped temperature; their results are not written
    const int b = col0 + n * 16 + li;
    const float T = temp[n];
    const bool greedy = row_is_greedy(T);
    const float inv_t = row_inv_temperature(T);
    static_for<MR>([&](auto m) FS_INLINE {
      if (Loop::owns(wave, m, n)) {
        const int v0 = row0 + m * 16 + 4 * kb;  // a multiple of 4
        push_four<ALIGN4>(best[n], acc[m][n], v0, a.V, static_cast<uint32_t>(a.vocab_offset + v0),
                          static_cast<uint32_t>(b), a.step, greedy, inv_t, philox);
      }
    });
  });
  // lanes l, l^16, l^32, l^48 hold the same batch row
  static_for<NT>([&](auto n) FS_INLINE {
    best[n].xor_reduce(16);
    best[n].xor_reduce(32);
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
  // block column c is covered by the waves w with col_off(w) == c - c % (NT*16)
  for (int c = threadIdx.x; c < Loop::kBlockCols; c += NW * kWave) {
    const int b = block_col0 + c;
    if (b >= a.B) break;
    ArgMax m;
    m.init();
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (Loop::col_off(w) == c - c % (NT * 16)) m.push(s_val[w][c % (NT * 16)], s_idx[w][c % (NT * 16)]);
    const size_t o = static_cast<size_t>(b) * a.S + blockIdx.x;
    a.part_val[o] = m.v;
    a.part_idx[o] = m.i;
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
// Requires D == 32 * NW * KS.
// ---------------------------------------------------------------------------
template <int NT, int NW, int KS, int P, bool ALIGN4>
__global__ __launch_bounds__(NW * kWave) void persist_sample_kernel(SampleArgs a) {
  static_assert(KS % P == 0, "the load ring must tile a group");
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  f32x4* red = reinterpret_cast<f32x4*>(dyn_smem);  // [2][NW][NT][kWave]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  const int D = a.D;
  const int kbeg = wave * KS * 32 + 8 * kb;
  const int ngroups = (a.V + 15) / 16;
  const int G = gridDim.x;

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

  auto group_ptr = [&](int g) FS_INLINE {
    return a.W + static_cast<size_t>(min(min(g, ngroups - 1) * 16 + li, a.V - 1)) * D + kbeg;
  };
  const Philox philox(a.seed);
  ArgMax best[NT];
  static_for<NT>([&](auto n) FS_INLINE { best[n].init(); });

  int g = blockIdx.x;
  const __bf16* ap = group_ptr(g);
  const __bf16* ap_next = group_ptr(g + G);
  bf16x8 ring[P];
  static_for<P>([&](auto p) FS_INLINE { ring[p] = load_frag(ap + p * 32); });

  for (int it = 0; g < ngroups; g += G, ++it) {
    f32x4 acc[NT];
    static_for<NT>([&](auto n) FS_INLINE { acc[n] = f32x4{0.f, 0.f, 0.f, 0.f}; });
    static_for<KS>([&](auto sc) FS_INLINE {
      constexpr int s = decltype(sc)::value;
      constexpr int slot = s % P;
      static_for<NT>([&](auto n) FS_INLINE { acc[n] = mfma16(ring[slot], hreg[s][n], acc[n]); });
      // refill with the k-step P ahead (the next group's, past the end of this one)
      if constexpr (s + P < KS)
        ring[slot] = load_frag(ap + (s + P) * 32);
      else
        ring[slot] = load_frag(ap_next + (s + P - KS) * 32);
    });
    ap = ap_next;
    ap_next = group_ptr(g + 2 * G);

    const int par = it & 1;
    static_for<NT>([&](auto n) FS_INLINE {
      red[((par * NW + wave) * NT + n) * kWave + lane] = acc[n];
    });
    __syncthreads();
    static_for<NT>([&](auto n) FS_INLINE {
      if ((n + it) % NW == wave && bvalid[n]) {
        f32x4 z = red[((par * NW + 0) * NT + n) * kWave + lane];
        for (int w = 1; w < NW; ++w) z += red[((par * NW + w) * NT + n) * kWave + lane];
        const int b = n * 16 + li;
        const int v0 = g * 16 + 4 * kb;  // ids grow with g for each owner
        push_four<ALIGN4>(best[n], z, v0, a.V, static_cast<uint32_t>(a.vocab_offset + v0),
                          static_cast<uint32_t>(b), a.step, greedy[n], inv_t[n], philox);
      }
    });
  }

  static_for<NT>([&](auto n) FS_INLINE {
    best[n].xor_reduce(16);
    best[n].xor_reduce(32);
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
}

// One wave per batch row: argmax over P (value, id) pairs.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ val,
                                                    const int32_t* __restrict__ idx,
                                                    int32_t P, int32_t B, int64_t stride_p,
                                                    int64_t stride_b, int32_t* out_ids,
                                                    float* out_val) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wave
  ArgMax m;
  m.init();
  for (int p = lane; p < P; p += kWave) {
    const int64_t o = p * stride_p + b * stride_b;
    m.push(val[o], idx[o]);
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) m.xor_reduce(mask);
  if (lane == 0) {
    out_ids[b] = m.i;
    out_val[b] = m.v;
  }
}

__global__ __launch_bounds__(256) void debug_noise_kernel(uint64_t seed, uint64_t step,
                                                          uint32_t row, uint32_t gv0,
                                                          int64_t n, uint32_t* bits,
                                                          float* g) {
  const Philox philox(seed);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const uint32_t gv = gv0 + static_cast<uint32_t>(i);
    const uint32_t x = pick_word(philox(noise_counter(gv, row, step)), gv & 3u);
    if (bits) bits[i] = x;
    if (g) g[i] = gumbel_from_bits(x);
  }
}

__global__ __launch_bounds__(256) void debug_gumbel_kernel(const uint32_t* bits, int64_t n,
                                                           float* g) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x)
    g[i] = gumbel_from_bits(bits[i]);
}

// ---------------------------------------------------------------------------
// Host side: configuration table and launchers.
// ---------------------------------------------------------------------------
namespace {

template <class Loop>
hipError_t launch_cfg(SampleArgs& a, hipStream_t stream) {
  constexpr int rows = Loop::kRowsPerBlock;
  static_assert(rows >= kMinRowsPerBlock, "split count bound");
  if (!Loop::supports(a.D) || static_cast<size_t>(a.B) * a.D * 2 > Loop::kMaxHBytes)
    return hipErrorInvalidValue;
  constexpr size_t smem = Loop::kSmemBytes;
  if (smem > 0) {  // may exceed the default dynamic-LDS limit: raise it once per kernel
    static const hipError_t attr = [] {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&fused_sample_kernel<Loop, true>),
          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
      if (e != hipSuccess) return e;
      return hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_sample_kernel<Loop, false>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(smem));
    }();
    if (attr != hipSuccess) return attr;
  }
  a.S = (a.V + rows - 1) / rows;
  const dim3 grid(a.S, (a.B + Loop::kBlockCols - 1) / Loop::kBlockCols);
  if (a.vocab_offset % 4 == 0)
    fused_sample_kernel<Loop, true><<<grid, Loop::NW * kWave, smem, stream>>>(a);
  else
    fused_sample_kernel<Loop, false><<<grid, Loop::NW * kWave, smem, stream>>>(a);
  return hipGetLastError();
}

template <class Loop>
bool supports_cfg(int32_t B, int32_t D) {
  return Loop::supports(D) && static_cast<size_t>(B) * D * 2 <= Loop::kMaxHBytes;
}

// Blocks of `kernel` that fit on one CU, times the CU count of the current
// device (cached per device).
template <class Kernel>
int resident_blocks(Kernel kernel, int threads, size_t smem) {
  static int cached_dev = -1, cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, smem) !=
            hipSuccess)
      return 0;
    cached = cus * (per_cu > 0 ? per_cu : 1);
    cached_dev = dev;
  }
  return cached;
}

template <int NT, int NW, int KS, int P>
struct Persist {
  static constexpr size_t kSmemBytes = 2ull * NW * NT * kWave * sizeof(f32x4);
  static bool supports(int32_t B, int32_t D) { return B <= NT * 16 && D == 32 * NW * KS; }
  static hipError_t launch(SampleArgs& a, hipStream_t stream) {
    if (!supports(a.B, a.D)) return hipErrorInvalidValue;
    const int ngroups = (a.V + 15) / 16;
    const bool al4 = a.vocab_offset % 4 == 0;
    const int slots = al4 ? resident_blocks(persist_sample_kernel<NT, NW, KS, P, true>,
                                            NW * kWave, kSmemBytes)
                          : resident_blocks(persist_sample_kernel<NT, NW, KS, P, false>,
                                            NW * kWave, kSmemBytes);
    if (slots <= 0) return hipErrorInvalidDevice;
    a.S = ngroups < slots ? ngroups : slots;
    if (al4)
      persist_sample_kernel<NT, NW, KS, P, true><<<a.S, NW * kWave, kSmemBytes, stream>>>(a);
    else
      persist_sample_kernel<NT, NW, KS, P, false><<<a.S, NW * kWave, kSmemBytes, stream>>>(a);
    return hipGetLastError();
  }
};

struct FusedConfig {
  const char* name;
  int rows_per_block;
  hipError_t (*launch)(SampleArgs&, hipStream_t);
  bool (*supports)(int32_t B, int32_t D);
  int order;  // configurations of equal order sum the contraction identically
};

template <class Loop>
constexpr FusedConfig make_cfg(const char* name, int order) {
  return {name, Loop::kRowsPerBlock, &launch_cfg<Loop>, &supports_cfg<Loop>, order};
}

template <class Pol>
constexpr FusedConfig make_persist(const char* name, int order) {
  return {name, 16, &Pol::launch, &Pol::supports, order};
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
#define FS_PERSIST(NT, NW, KS, P) \
  make_persist<Persist<NT, NW, KS, P>>("persist_nt" #NT "_nw" #NW "_ks" #KS "_p" #P, 100 + NW)

const FusedConfig kConfigs[] = {
    FS_KSPLIT(1, 1, 4, 8, 0),           // 0  B <= 8 when no persistent shape fits
    FS_LDS(2, 4, 4, 64, 4, 0),          // 1  B <= 64 when 14 would leave CUs idle
    FS_DMAG(4, 8, 8, 64, 4, 3, 4, 2),   // 2  B <= 128
    FS_DMAG(2, 16, 8, 64, 4, 4, 4, 2),  // 3  B > 128 (batch blocks of 256)
    FS_STREAM(4, 1, 4, 4, 0),           // 4  any D: fallback for B <= 16
    FS_STREAM(2, 4, 4, 4, 0),           // 5  any D: fallback for larger B
    FS_PERSIST(1, 8, 16, 8),            // 6  D = 4096, B <= 16
    FS_PERSIST(2, 8, 16, 8),            // 7  D = 4096, B <= 32
    FS_PERSIST(1, 8, 32, 8),            // 8  D = 8192, B <= 16
    FS_PERSIST(1, 4, 2, 2),             // 9  D = 256 (small shapes)
    FS_PERSIST(2, 4, 2, 2),             // 10 D = 256
    FS_LDS(2, 16, 4, 64, 4, 0),         // 11 B > 128 when 2*B*D >= 2^31
    FS_LDSR(2, 16, 4, 64, 4, 1, 4),     // 12 B > 128 when 3 would leave CUs idle
    FS_LDSR(4, 8, 4, 64, 4, 1, 4),      // 13 B <= 128 when 2 would leave CUs idle
    FS_DMAG(4, 4, 8, 64, 4, 3, 4, 2),   // 14 B <= 64
    // alternatives for tuning sweeps
    FS_PERSIST(1, 8, 16, 16),
    FS_LDS(2, 8, 4, 64, 8, 0),
    FS_LDSR(2, 8, 4, 64, 8, 1, 4),
    FS_DMA(2, 16, 8, 64, 4, 4, 4),
    FS_DMA(4, 8, 8, 64, 4, 3, 4),
    FS_DMAG(2, 16, 8, 64, 8, 3, 4, 2),
    FS_DMAG(2, 8, 8, 64, 4, 4, 4, 2),
    FS_DMAG(2, 16, 8, 128, 4, 2, 4, 2),
    FS_KSPLIT(2, 1, 4, 8, 0),
    FS_KSPLIT(4, 2, 4, 4, 0),
    FS_STREAM(1, 1, 4, 8, 0),
};
#undef FS_STREAM
#undef FS_KSPLIT
#undef FS_LDS
#undef FS_PERSIST
#undef FS_LDSR
#undef FS_DMA
#undef FS_DMAG

constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace

int num_fused_configs() { return kNumConfigs; }

const char* fused_config_name(int id) {
  return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : nullptr;
}

int fused_rows_per_block(int id) {
  return (id >= 0 && id < kNumConfigs) ? kConfigs[id].rows_per_block : 0;
}

int fused_config_order(int id) {
  return (id >= 0 && id < kNumConfigs) ? kConfigs[id].order : -1;
}

bool fused_config_supports(int id, int32_t B, int32_t D) {
  return id >= 0 && id < kNumConfigs && kConfigs[id].supports(B, D);
}

namespace {
int device_cus() {
  static int cached_dev = -1, cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cached_dev) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached = cus;
    cached_dev = dev;
  }
  return cached;
}

// Share of CU slots busy over the whole grid of a configuration that runs one
// block per CU: blocks / (rounds * CUs).  A grid whose last round is mostly
// empty wastes that round.
double one_per_cu_fill(int id, int32_t V) {
  const int cus = device_cus();
  if (cus <= 0) return 0.0;
  const int rows = kConfigs[id].rows_per_block;
  const long blocks = (static_cast<long>(V) + rows - 1) / rows;
  const long rounds = (blocks + cus - 1) / cus;
  return static_cast<double>(blocks) / (static_cast<double>(rounds) * cus);
}
}  // namespace

int fused_auto_config(int32_t B, int32_t D, int32_t V) {
  // persistent K-split where h fits in registers
  for (int id : {6, 7, 8})
    if (kConfigs[id].supports(B, D)) return id;
  if (B <= 8 && kConfigs[0].supports(B, D)) return 0;
  // batch-tiled loops: the DMA-staged loop (one 8-wave block per CU) when its
  // grid fills the CUs, else the LDS loop (smaller blocks, two per CU)
  struct Pick { int dma, lds; };
  const Pick p = B <= 64 ? Pick{14, 1} : (B <= 128 ? Pick{2, 13} : Pick{3, 12});
  constexpr double kMinFill = 0.85;
  if (kConfigs[p.dma].supports(B, D) && one_per_cu_fill(p.dma, V) >= kMinFill) return p.dma;
  if (kConfigs[p.lds].supports(B, D)) return p.lds;
  if (B > 64 && kConfigs[11].supports(B, D)) return 11;
  return B <= 16 ? 4 : 5;
}

hipError_t launch_fused(int id, SampleArgs& a, hipStream_t stream) {
  return kConfigs[id].launch(a, stream);
}

hipError_t launch_merge(const float* val, const int32_t* idx, int32_t P, int32_t B,
                        int64_t stride_p, int64_t stride_b, int32_t* out_ids,
                        float* out_val, hipStream_t stream) {
  const dim3 grid((B + 3) / 4);
  merge_kernel<<<grid, 256, 0, stream>>>(val, idx, P, B, stride_p, stride_b, out_ids,
                                         out_val);
  return hipGetLastError();
}

hipError_t launch_debug_noise(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0,
                              int64_t n, uint32_t* bits, float* g, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
  debug_noise_kernel<<<grid, 256, 0, stream>>>(seed, step, row, gv0, n, bits, g);
  return hipGetLastError();
}

hipError_t launch_debug_gumbel(const uint32_t* bits, int64_t n, float* g,
                               hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
  debug_gumbel_kernel<<<grid, 256, 0, stream>>>(bits, n, g);
  return hipGetLastError();
}

}  // namespace fs
