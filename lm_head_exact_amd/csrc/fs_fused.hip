// fs_fused.hip -- the fused LM-head + Gumbel-Max sampler and the merge.
//
// FlashSampling (wiki summary, "Method"; arXiv abstract): compute each
// vocabulary tile's logits on chip, scale by 1/T, add per-element Gumbel
// noise, keep one (max, argmax) pair per row and per tile, and finish with a
// small reduction over tiles.  Because the argmax of logits plus noise
// decomposes over any partition of the vocabulary ("Key claims"), the result
// equals one global argmax over the full noise field.
//
// Grid: x = vocabulary blocks of NW * MR * 16 rows, y = batch blocks of
// NT * 16 rows.  Each wave owns MR * 16 consecutive vocabulary rows and all
// NT * 16 batch rows of its block, so every W element is read by one wave
// exactly once.  The epilogue runs in registers on the MFMA accumulators;
// the block writes one partial per batch row to part_[val|idx][b][block].
#include "fs_internal.hpp"
#include "fs_mma.hpp"

namespace fs {

template <int MR, int NT, int NW, bool ALIGN4>
__global__ __launch_bounds__(NW * kWave) void fused_sample_kernel(SampleArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  const int row0 = (blockIdx.x * NW + wave) * (MR * 16);
  const int col0 = blockIdx.y * (NT * 16);

  f32x4 acc[MR][NT];
  mma_block<MR, NT>(a.W, a.h, a.B, a.D, a.V, row0, col0, acc);

  // ---- epilogue: scale, perturb, running (max, argmax) per batch row ----
  const Philox philox(a.seed);
  ArgMax best[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    best[n].init();
    const int b = col0 + n * 16 + li;
    if (b >= a.B) continue;
    const float T = a.temperature[b];
    const bool greedy = row_is_greedy(T);
    const float inv_t = row_inv_temperature(T);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int v0 = row0 + m * 16 + 4 * kb;  // a multiple of 4
      const uint32_t gv0 = static_cast<uint32_t>(a.vocab_offset + v0);
      u32x4 words = u32x4{0u, 0u, 0u, 0u};
      if (ALIGN4 && !greedy) words = philox(noise_counter(gv0, b, a.step));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (v0 + r >= a.V) break;
        const uint32_t gv = gv0 + r;
        float s = acc[m][n][r];
        if (!greedy) {
          const uint32_t x = ALIGN4 ? pick_word(words, r)
                                    : pick_word(philox(noise_counter(gv, b, a.step)), gv & 3u);
          s = perturbed_score(s, inv_t, gumbel_from_bits(x));
        }
        best[n].push(s, static_cast<int32_t>(gv));
      }
    }
  }
  // lanes l, l^16, l^32, l^48 hold the same batch row
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    best[n].xor_reduce(16);
    best[n].xor_reduce(32);
  }

  __shared__ float s_val[NW][NT * 16];
  __shared__ int32_t s_idx[NW][NT * 16];
  if (kb == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      s_val[wave][n * 16 + li] = best[n].v;
      s_idx[wave][n * 16 + li] = best[n].i;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < NT * 16; c += NW * kWave) {
    const int b = col0 + c;
    if (b >= a.B) break;
    ArgMax m;
    m.init();
#pragma unroll
    for (int w = 0; w < NW; ++w) m.push(s_val[w][c], s_idx[w][c]);
    const size_t o = static_cast<size_t>(b) * a.S + blockIdx.x;
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

template <int MR, int NT, int NW>
hipError_t launch_cfg(SampleArgs& a, hipStream_t stream) {
  constexpr int rows = MR * 16 * NW;
  static_assert(rows >= kMinRowsPerBlock, "split count bound");
  a.S = (a.V + rows - 1) / rows;
  const dim3 grid(a.S, (a.B + NT * 16 - 1) / (NT * 16));
  if (a.vocab_offset % 4 == 0)
    fused_sample_kernel<MR, NT, NW, true><<<grid, NW * kWave, 0, stream>>>(a);
  else
    fused_sample_kernel<MR, NT, NW, false><<<grid, NW * kWave, 0, stream>>>(a);
  return hipGetLastError();
}

struct FusedConfig {
  const char* name;
  int rows_per_block;
  hipError_t (*launch)(SampleArgs&, hipStream_t);
};

#define FS_CFG(MR, NT, NW) \
  {"direct_mr" #MR "_nt" #NT "_nw" #NW, MR * 16 * NW, &launch_cfg<MR, NT, NW>}

const FusedConfig kConfigs[] = {
    FS_CFG(4, 1, 4),   // 0: B <= 16
    FS_CFG(4, 2, 4),   // 1: B <= 32
    FS_CFG(2, 4, 4),   // 2: B <= 64
    FS_CFG(1, 8, 4),   // 3: B <= 128
    FS_CFG(1, 16, 4),  // 4: B > 128 (batch blocks of 256)
    FS_CFG(2, 1, 4),   // 5: alternatives for tuning sweeps
    FS_CFG(2, 2, 4),   // 6
};
#undef FS_CFG

constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace

int num_fused_configs() { return kNumConfigs; }

const char* fused_config_name(int id) {
  return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : nullptr;
}

int fused_rows_per_block(int id) {
  return (id >= 0 && id < kNumConfigs) ? kConfigs[id].rows_per_block : 0;
}

int fused_auto_config(int32_t B, int32_t /*D*/, int32_t /*V*/) {
  if (B <= 16) return 0;
  if (B <= 32) return 1;
  if (B <= 64) return 2;
  if (B <= 128) return 3;
  return 4;
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
