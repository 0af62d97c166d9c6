// fs_online.hip -- the online (chunked) sampler with early finalisation.
//
// In the online setting the vocabulary is consumed as consecutive pieces and
// the running Gumbel-max over the pieces seen so far is the sample over them
// (wiki summary, "Method", last paragraph: the sampler streams over
// vocabulary pieces and may finalise early).  Each chunk here is one fused
// sampler launch over W's rows [cuts[c], cuts[c+1]); a step kernel then folds
// the chunk's tile partials into every live row's running (max, argmax).
//
// The pages give no stopping bound; this one follows from Cauchy-Schwarz.  A
// later logit obeys z = h_b . W_v <= |h_b| R_c, with R_c the largest row norm
// of the chunks after c, and a noise value is at most g_max, the largest
// value of the Gumbel map (at the top word).  Row b is therefore final
// after chunk c when its running best exceeds
//     (|h_b| R_c (1/T) + g_max) (1 + 2^-8)      (greedy rows: |h_b| R_c (1 + 2^-8)).
// The factor 1 + 2^-8 covers the rounding of the device's fp32 logits (at
// most ~D 2^-24 relative, so D <= 32768), scores and Gumbel values: every
// score a later chunk could produce on the device stays below the bound, and
// stopping never changes the sample.
//
// Once no row is live, the later chunks' sampler blocks and steps return at
// once (SampleArgs::live), so their W rows are never read.  Norms are fp64.
#include "fs_device.hpp"
#include "fs_internal.hpp"

namespace fs {

namespace {

// Euclidean norm of one bf16 row of length D (D % 8 == 0, 16-byte aligned),
// summed by one wave in fp64 and returned in every lane.
__device__ __forceinline__ double wave_row_norm(const __bf16* x, int32_t D, int lane) {
  double s = 0.0;
  for (int d = lane * 8; d < D; d += kWave * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(x + d);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = __uint_as_float(w[j] << 16);
      const double hi = __uint_as_float(w[j] & 0xFFFF0000u);
      s += lo * lo;
      s += hi * hi;
    }
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask, kWave);
  return sqrt(s);
}

// One wave per row.
__global__ __launch_bounds__(256) void row_norms_kernel(const __bf16* __restrict__ X, int32_t n,
                                                        int32_t D, double* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = blockIdx.x * 4ll + (threadIdx.x >> 6);
  if (r >= n) return;  // uniform per wave
  const double nrm = wave_row_norm(X + r * D, D, lane);
  if (lane == 0) out[r] = nrm;
}

// One wave per 16-row group of fragment-order W (packed_frag's layout): lane l
// sums the squares of its 16-byte pieces over the group's k-steps (1 KB
// contiguous per step), and the four lanes l, l ^ 16, l ^ 32, l ^ 48 that hold
// the same row combine their sums; rows outside [0, V) (padding) are skipped.
__global__ __launch_bounds__(256) void packed_row_norms_kernel(const __bf16* __restrict__ Wp,
                                                               int32_t V, int32_t D, int32_t shift,
                                                               int64_t groups,
                                                               double* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t g = blockIdx.x * 4ll + (threadIdx.x >> 6);
  if (g >= groups) return;  // uniform per wave
  const int ksteps = D / 32;
  const __bf16* p = Wp + (g * ksteps * kWave + lane) * 8;
  double s = 0.0;
  for (int k = 0; k < ksteps; ++k) {
    const uint4 q = *reinterpret_cast<const uint4*>(p + static_cast<int64_t>(k) * kWave * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = __uint_as_float(w[j] << 16);
      const double hi = __uint_as_float(w[j] & 0xFFFF0000u);
      s += lo * lo;
      s += hi * hi;
    }
  }
  s += __shfl_xor(s, 16, kWave);
  s += __shfl_xor(s, 32, kWave);
  const int64_t v = g * 16 + (lane & 15) - shift;
  if (lane < 16 && v >= 0 && v < V) out[v] = sqrt(s);
}

// One block: out[0] = max(x[0 .. n)) of non-negative values (0 if n == 0).
__global__ __launch_bounds__(256) void max_reduce_kernel(const double* __restrict__ x, int32_t n,
                                                         double* __restrict__ out) {
  __shared__ double s_max[256];
  double m = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) m = fmax(m, x[i]);
  s_max[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w)
      s_max[threadIdx.x] = fmax(s_max[threadIdx.x], s_max[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = s_max[0];
}

// One thread: later[c] = max over the chunks after c.
__global__ __launch_bounds__(64) void suffix_max_kernel(const double* __restrict__ chunk_max,
                                                        int32_t n_chunks,
                                                        double* __restrict__ later) {
  if (threadIdx.x != 0) return;
  double m = 0.0;
  for (int c = n_chunks - 1; c >= 0; --c) {
    later[c] = m;
    m = fmax(m, chunk_max[c]);
  }
}

// One wave per batch row: |h_b|, the running pair (-inf, INT32_MAX), chunk
// count 0, not final; block 0 clears the live counts of every chunk.
__global__ __launch_bounds__(256) void online_init_kernel(
    const __bf16* __restrict__ h, int32_t B, int32_t D, int32_t n_chunks,
    double* __restrict__ hnorm, int32_t* __restrict__ done, int32_t* __restrict__ live,
    int32_t* __restrict__ out_ids, float* __restrict__ out_val, int32_t* __restrict__ out_chunks) {
  if (blockIdx.x == 0)
    for (int c = threadIdx.x; c < n_chunks; c += 256) live[c] = 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wave
  const double nrm = wave_row_norm(h + static_cast<int64_t>(b) * D, D, lane);
  if (lane == 0) {
    hnorm[b] = nrm;
    done[b] = 0;
    out_ids[b] = 0x7FFFFFFF;
    out_val[b] = -__builtin_inff();
    out_chunks[b] = 0;
  }
}

// One wave per batch row (element (b, t) of the chunk's partials at b * S + t).
__global__ __launch_bounds__(256) void online_step_kernel(
    const float* __restrict__ part_val, const int32_t* __restrict__ part_idx, int32_t S,
    int32_t B, int32_t c, int32_t n_chunks, const double* __restrict__ later,
    const double* __restrict__ hnorm, const float* __restrict__ temperature, double g_max,
    double margin, int32_t* __restrict__ done, int32_t* live, int32_t* __restrict__ out_ids,
    float* __restrict__ out_val, int32_t* __restrict__ out_chunks) {
  if (c > 0 && live[c - 1] == 0) return;  // every row was final: chunk c was not sampled
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B || done[b] != 0) return;  // uniform per wave
  ArgMax m;
  m.init();
  if (lane == 0) {  // the running pair: its ids precede the chunk's
    m.v = out_val[b];
    m.i = out_ids[b];
  }
  strided_argmax(part_val, part_idx, S, lane,
                 [&](int t) FS_INLINE { return static_cast<int64_t>(b) * S + t; }, m);
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) m.xor_reduce(mask);
  if (lane == 0) {
    out_val[b] = m.v;
    out_ids[b] = m.i;
    out_chunks[b] = c + 1;
    bool final_row = false;
    if (c + 1 < n_chunks) {
      const float T = temperature[b];
      const bool greedy = row_is_greedy(T);
      const double reach = hnorm[b] * later[c];
      const double bound = greedy ? reach * margin
                                  : (reach * static_cast<double>(row_inv_temperature(T)) + g_max) *
                                        margin;
      final_row = static_cast<double>(m.v) > bound;
    }
    if (final_row)
      done[b] = 1;
    else
      atomicAdd(live + c, 1);
  }
}

}  // namespace

hipError_t launch_row_norms(const __bf16* X, int32_t n, int32_t D, double* out,
                            hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  row_norms_kernel<<<dim3((n + 3) / 4), 256, 0, stream>>>(X, n, D, out);
  return hipGetLastError();
}

hipError_t launch_packed_row_norms(const __bf16* Wp, int32_t V, int32_t D, int32_t vocab_offset,
                                   double* out, hipStream_t stream) {
  const int64_t groups = packed_groups(V, vocab_offset);
  packed_row_norms_kernel<<<dim3(static_cast<unsigned>((groups + 3) / 4)), 256, 0, stream>>>(
      Wp, V, D, vocab_offset & 3, groups, out);
  return hipGetLastError();
}

hipError_t launch_max_reduce(const double* x, int32_t n, double* out, hipStream_t stream) {
  max_reduce_kernel<<<1, 256, 0, stream>>>(x, n, out);
  return hipGetLastError();
}

hipError_t launch_suffix_max(const double* chunk_max, int32_t n_chunks, double* later,
                             hipStream_t stream) {
  suffix_max_kernel<<<1, 64, 0, stream>>>(chunk_max, n_chunks, later);
  return hipGetLastError();
}

hipError_t launch_online_init(const __bf16* h, int32_t B, int32_t D, int32_t n_chunks,
                              double* hnorm, int32_t* done, int32_t* live, int32_t* out_ids,
                              float* out_val, int32_t* out_chunks, hipStream_t stream) {
  online_init_kernel<<<dim3((B + 3) / 4), 256, 0, stream>>>(h, B, D, n_chunks, hnorm, done, live,
                                                            out_ids, out_val, out_chunks);
  return hipGetLastError();
}

hipError_t launch_online_step(const float* part_val, const int32_t* part_idx, int32_t S,
                              int32_t B, int32_t c, int32_t n_chunks, const double* later,
                              const double* hnorm, const float* temperature, double g_max,
                              double margin, int32_t* done, int32_t* live, int32_t* out_ids,
                              float* out_val, int32_t* out_chunks, hipStream_t stream) {
  online_step_kernel<<<dim3((B + 3) / 4), 256, 0, stream>>>(
      part_val, part_idx, S, B, c, n_chunks, later, hnorm, temperature, g_max, margin, done, live,
      out_ids, out_val, out_chunks);
  return hipGetLastError();
}

}  // namespace fs
