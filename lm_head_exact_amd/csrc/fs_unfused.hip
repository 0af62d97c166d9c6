// fs_unfused.hip -- the standard unfused decode-step sampler, as a baseline.
//
// The four back-to-back operations the FlashSampling pages describe as the
// usual decode step (wiki summary, "Method", first paragraph): the LM-head
// matmul writes the B x V logits to device memory; a softmax pass reads them
// back; Gumbel perturbation and the argmax read them once more.  Every pass
// after the matmul is a bandwidth-bound sweep over B x V values, which is the
// traffic the fused kernel removes.
//
// Kernels (all on the caller's stream):
//   1. gemm_logits     z[b][v] (fp32, row stride ldz)   -- same MFMA main loop
//   2. softmax_stats   per (row, chunk): max and sum of exp(z/T - max)
//   3. softmax_probs   p[b][v] = exp(z/T - lse_b), lse_b from the chunk stats
//   4. gumbel_argmax   per (row, chunk): argmax of log p + g (+ lse_b), or of
//                      z for greedy rows
//   5. merge           argmax over the chunks (shared with the fused path)
// The noise field is the same Philox/Gumbel field as the fused sampler, so
// both return the same ids up to fp32 rounding.
#include "fs_internal.hpp"
#include "fs_mma.hpp"

namespace fs {
namespace {

constexpr int kChunk = 4096;  // vocabulary entries per (row, chunk) block
constexpr int kThreads = 256;

struct UnfusedLayout {
  int64_t ldz;  // row stride of the logits / probability matrices
  int32_t C;    // chunks per row
  float* logits;
  float* probs;
  float2* stats;  // [B][C] (max, sum)
  float* lse;     // [B]
  float* part_val;
  int32_t* part_idx;  // [B][C]
};

UnfusedLayout layout(int32_t B, int32_t V, void* ws) {
  UnfusedLayout L;
  L.ldz = static_cast<int64_t>(round_up(static_cast<size_t>(V), 64));
  L.C = (V + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = p;
    p += round_up(bytes, 256);
    return r;
  };
  L.logits = reinterpret_cast<float*>(take(sizeof(float) * B * L.ldz));
  L.probs = reinterpret_cast<float*>(take(sizeof(float) * B * L.ldz));
  L.stats = reinterpret_cast<float2*>(take(sizeof(float2) * B * L.C));
  L.lse = reinterpret_cast<float*>(take(sizeof(float) * B));
  L.part_val = reinterpret_cast<float*>(take(sizeof(float) * B * L.C));
  L.part_idx = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * L.C));
  return L;
}

// logits z[b][v] for a (Loop::kRowsPerBlock x Loop::kBlockCols) tile per
// block, with the same main loops as the fused sampler.
template <class Loop>
__global__ __launch_bounds__(Loop::NW * kWave)
__attribute__((amdgpu_waves_per_eu(Loop::kWavesPerSimd))) void gemm_logits_kernel(SampleArgs a,
                                                                                  float* z,
                                                                                  int64_t ldz) {
  constexpr int MR = Loop::MR, NT = Loop::NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_smem[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15, kb = lane >> 4;
  const int row0 = Loop::row0(blockIdx.x, wave);
  const int block_col0 = blockIdx.y * Loop::kBlockCols;
  f32x4 acc[MR][NT];
  Loop::run(a.W, a.h, a.B, a.D, a.V, row0, block_col0, acc, dyn_smem);
  const int col0 = block_col0 + Loop::col_off(wave);
  static_for<NT>([&](auto n) FS_INLINE {
    const int b = col0 + n * 16 + li;
    if (b < a.B) {
      static_for<MR>([&](auto m) FS_INLINE {
        if (Loop::owns(wave, m, n)) {
          const int v0 = row0 + m * 16 + 4 * kb;
          float* dst = z + b * ldz + v0;
          if (v0 + 3 < a.V) {
            *reinterpret_cast<f32x4*>(dst) = acc[m][n];  // ldz % 4 == 0, v0 % 4 == 0
          } else {
            static_for<4>([&](auto r) FS_INLINE {
              if (v0 + r < a.V) dst[r] = acc[m][n][decltype(r)::value];
            });
          }
        }
      });
    }
  });
}

template <class Loop>
hipError_t launch_gemm(const SampleArgs& a, float* z, int64_t ldz, hipStream_t stream) {
  constexpr size_t smem = Loop::kSmemBytes;
  if (smem > 0) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_logits_kernel<Loop>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (attr != hipSuccess) return attr;
  }
  const dim3 grid((a.V + Loop::kRowsPerBlock - 1) / Loop::kRowsPerBlock,
                  (a.B + Loop::kBlockCols - 1) / Loop::kBlockCols);
  gemm_logits_kernel<Loop><<<grid, Loop::NW * kWave, smem, stream>>>(a, z, ldz);
  return hipGetLastError();
}

// Block-wide reductions over kThreads threads.
__device__ float block_max(float x, float* sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, sh[i]);
  return r;
}

__device__ float block_sum(float x, float* sh) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r += sh[i];
  return r;
}

// grid (C, B): chunk statistics of s = z / T.
__global__ __launch_bounds__(kThreads) void softmax_stats_kernel(const float* z, int64_t ldz,
                                                                 int32_t V,
                                                                 const float* temperature,
                                                                 float2* stats, int32_t C) {
  __shared__ float sh[kThreads / kWave];
  const int b = blockIdx.y, c = blockIdx.x;
  const float T = temperature[b];
  if (row_is_greedy(T)) return;  // greedy rows skip the softmax
  const float inv_t = row_inv_temperature(T);
  const int v_begin = c * kChunk, v_end = min(V, v_begin + kChunk);
  const float* zr = z + b * ldz;
  float m = -__builtin_inff();
  for (int v = v_begin + threadIdx.x; v < v_end; v += kThreads) m = fmaxf(m, zr[v] * inv_t);
  m = block_max(m, sh);
  float l = 0.f;
  for (int v = v_begin + threadIdx.x; v < v_end; v += kThreads) l += expf(zr[v] * inv_t - m);
  l = block_sum(l, sh);
  if (threadIdx.x == 0) stats[static_cast<int64_t>(b) * C + c] = make_float2(m, l);
}

// grid (C, B): p = exp(z / T - lse), lse combined from the chunk statistics.
__global__ __launch_bounds__(kThreads) void softmax_probs_kernel(
    const float* z, float* p, int64_t ldz, int32_t V, const float* temperature,
    const float2* stats, int32_t C, float* lse_out) {
  __shared__ float sh[kThreads / kWave];
  const int b = blockIdx.y, c = blockIdx.x;
  const float T = temperature[b];
  if (row_is_greedy(T)) return;
  const float inv_t = row_inv_temperature(T);
  float m = -__builtin_inff();
  for (int i = threadIdx.x; i < C; i += kThreads) m = fmaxf(m, stats[static_cast<int64_t>(b) * C + i].x);
  m = block_max(m, sh);
  float l = 0.f;
  for (int i = threadIdx.x; i < C; i += kThreads) {
    const float2 st = stats[static_cast<int64_t>(b) * C + i];
    l += st.y * expf(st.x - m);
  }
  l = block_sum(l, sh);
  const float lse = m + logf(l);
  if (c == 0 && threadIdx.x == 0) lse_out[b] = lse;
  const int v_begin = c * kChunk, v_end = min(V, v_begin + kChunk);
  const float* zr = z + b * ldz;
  float* pr = p + b * ldz;
  for (int v = v_begin + threadIdx.x; v < v_end; v += kThreads) pr[v] = expf(zr[v] * inv_t - lse);
}

// grid (C, B): per-chunk argmax of log p + g (scores reported on the
// z / T + g scale by adding lse back), or of z for greedy rows.
__global__ __launch_bounds__(kThreads) void gumbel_argmax_kernel(
    const float* z, const float* p, int64_t ldz, int32_t V, int32_t vocab_offset,
    const float* temperature, const float* lse, uint64_t seed, uint64_t step,
    float* part_val, int32_t* part_idx, int32_t C) {
  __shared__ float s_v[kThreads / kWave];
  __shared__ int32_t s_i[kThreads / kWave];
  const int b = blockIdx.y, c = blockIdx.x;
  const float T = temperature[b];
  const bool greedy = row_is_greedy(T);
  const float row_lse = greedy ? 0.f : lse[b];
  const Philox philox(seed);
  const int v_begin = c * kChunk, v_end = min(V, v_begin + kChunk);
  ArgMax best;
  best.init();
  for (int v = v_begin + threadIdx.x; v < v_end; v += kThreads) {
    const uint32_t gv = static_cast<uint32_t>(vocab_offset + v);
    float s;
    if (greedy) {
      s = z[b * ldz + v];
    } else {
      const uint32_t x = pick_word(philox(noise_counter(gv, b, step)), gv & 3u);
      s = __fadd_rn(__fadd_rn(logf(p[b * ldz + v]), gumbel_from_bits(x)), row_lse);
    }
    best.push(s, static_cast<int32_t>(gv));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best.xor_reduce(m);
  if ((threadIdx.x & 63) == 0) {
    s_v[threadIdx.x >> 6] = best.v;
    s_i[threadIdx.x >> 6] = best.i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgMax r;
    r.init();
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) r.push(s_v[w], s_i[w]);
    part_val[static_cast<int64_t>(b) * C + c] = r.v;
    part_idx[static_cast<int64_t>(b) * C + c] = r.i;
  }
}

}  // namespace

size_t unfused_workspace_bytes(int32_t B, int32_t V) {
  const size_t ldz = round_up(static_cast<size_t>(V), 64);
  const size_t C = (static_cast<size_t>(V) + kChunk - 1) / kChunk;
  const size_t rows = static_cast<size_t>(B);
  return round_up(sizeof(float) * rows * ldz, 256) * 2 + round_up(sizeof(double) * rows * C, 256) +
         round_up(sizeof(float) * rows, 256) + round_up(sizeof(float) * rows * C, 256) * 2;
}

hipError_t launch_unfused(const SampleArgs& a, int32_t* out_ids, float* out_val,
                          void* workspace, hipStream_t stream) {
  const UnfusedLayout L = layout(a.B, a.V, workspace);
  {
    // the contraction with the fused sampler's main loops: W read once per
    // batch block of 32 (streamed) or 256 (h staged in LDS) rows
    using Big = LdsLoop<2, 16, 4, 64, 4, false, 1, 4>;
    const hipError_t e = a.B > 32 && Big::supports(a.D)
                             ? launch_gemm<Big>(a, L.logits, L.ldz, stream)
                             : launch_gemm<StreamLoop<2, 2, 4, 4, false>>(a, L.logits, L.ldz, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 rows(L.C, a.B);
  softmax_stats_kernel<<<rows, kThreads, 0, stream>>>(L.logits, L.ldz, a.V, a.temperature,
                                                      L.stats, L.C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  softmax_probs_kernel<<<rows, kThreads, 0, stream>>>(L.logits, L.probs, L.ldz, a.V,
                                                      a.temperature, L.stats, L.C, L.lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  gumbel_argmax_kernel<<<rows, kThreads, 0, stream>>>(L.logits, L.probs, L.ldz, a.V,
                                                      a.vocab_offset, a.temperature, L.lse,
                                                      a.seed, a.step, L.part_val, L.part_idx,
                                                      L.C);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(L.part_val, L.part_idx, L.C, a.B, 1, L.C, out_ids, out_val, stream);
}

}  // namespace fs
