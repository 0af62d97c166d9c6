// fs_device.hpp -- device building blocks of libflashsample (gfx950).
//
// Counter-based noise, the uniform -> Gumbel map, the (max, argmax)
// comparator and wave-level reductions shared by the fused sampler, the
// unfused baseline and the diagnostics.  Written for CDNA4: 64-lane
// wavefronts, bf16 MFMA operand vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>).  Register
// arrays (accumulators, per-row maxima) are only indexed with these constants,
// so they never fall back to scratch memory whatever the unroller decides.
// Loop bodies are lambdas marked FS_INLINE: a body left as a call would force
// the arrays it captures into addressable (scratch) memory.
#define FS_INLINE __attribute__((always_inline))
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each round multiplies
// counter words 0 and 2 by two fixed odd 32-bit constants; the high halves,
// xored with the other two words and the round key, and the low halves form
// the next counter.  The key advances by two Weyl increments per round.  The
// key words are uniform across the wave, so the compiler keeps the schedule
// in scalar registers.
// ---------------------------------------------------------------------------
struct Philox {
  uint32_t k0, k1;

  __device__ __forceinline__ explicit Philox(uint64_t seed)
      : k0(static_cast<uint32_t>(seed)), k1(static_cast<uint32_t>(seed >> 32)) {}

  __device__ __forceinline__ u32x4 operator()(u32x4 c) const {
    uint32_t a = k0, b = k1;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      const uint64_t p = static_cast<uint64_t>(0xD2511F53u) * c.x;
      const uint64_t q = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
      const uint32_t p_hi = static_cast<uint32_t>(p >> 32), p_lo = static_cast<uint32_t>(p);
      const uint32_t q_hi = static_cast<uint32_t>(q >> 32), q_lo = static_cast<uint32_t>(q);
      // three-input xors as single v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
      const uint32_t c0 = static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(q_hi, c.y, a, 0x96));
      const uint32_t c2 = static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(p_hi, c.w, b, 0x96));
      c = u32x4{c0, q_lo, c2, p_lo};
      a += 0x9E3779B9u;
      b += 0xBB67AE85u;
    }
    return c;
  }
};

// Counter of the block that holds global id gv for batch row `row`: one
// block serves the four ids 4m .. 4m+3 (word gv mod 4).
__device__ __forceinline__ u32x4 noise_counter(uint32_t gv, uint32_t row, uint64_t step) {
  return u32x4{gv >> 2, row, static_cast<uint32_t>(step), static_cast<uint32_t>(step >> 32)};
}

__device__ __forceinline__ uint32_t pick_word(u32x4 w, uint32_t i) {
  return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// Standard Gumbel value of a 32-bit word x: u = (x + 1/2) 2^-32, the midpoint
// of the word's cell (all 32 bits count), and g = -ln(-ln u).
//
// Cost matters: this runs once per logit of the B x V tile, so it uses the
// hardware base-2 logarithm (v_log_f32) instead of the library's
// extended-precision logf/log1pf (about ten times the instructions).  The
// one place where that is not accurate enough is -ln u for u near 1, where
// the winners of a large vocabulary sit (u ~ 1 - 1/V): there ln u is a small
// difference and an absolute error in log2 u becomes a large relative error
// in -ln u, which the outer log turns into an absolute error in g.  So both
// u and v = 1 - u are formed from the word itself, v from its complement:
// v = (~x + 1/2) 2^-32.  Each is one conversion and one fused multiply-add,
// within 2^-23 relative of the exact value (exact for ~x < 2^23, where the
// largest scores of a big vocabulary come from).  For v <= 1/16 the series
// -ln(1 - v) = v + v^2/2 + ... + v^5/5 (truncation below 1.6e-7 relative)
// gives -ln u; elsewhere |ln u| >= 0.06 and the hardware log of u is used.
// Checked against the fp64 oracle on the top 2^24 and bottom 2^20 words and
// on a stratified grid of the rest.
__device__ __forceinline__ float gumbel_from_bits(uint32_t x) {
  constexpr float kLn2 = 0.693147180559945309f;
  const float u = __builtin_fmaf(static_cast<float>(x), 0x1p-32f, 0x1p-33f);
  const float v = __builtin_fmaf(static_cast<float>(~x), 0x1p-32f, 0x1p-33f);
  float series = 1.0f / 5.0f;
  series = __builtin_fmaf(series, v, 1.0f / 4.0f);
  series = __builtin_fmaf(series, v, 1.0f / 3.0f);
  series = __builtin_fmaf(series, v, 1.0f / 2.0f);
  series = __builtin_fmaf(series, v, 1.0f);
  series *= v;
  const float neg_ln_u = v <= 0.0625f ? series : -__builtin_amdgcn_logf(u) * kLn2;
  return -__builtin_amdgcn_logf(neg_ln_u) * kLn2;
}

// ---------------------------------------------------------------------------
// (value, id) maximum with ties to the smaller id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi) {
  return v > bv || (v == bv && i < bi);
}

struct ArgMax {
  float v;
  int32_t i;
  __device__ __forceinline__ void init() {
    v = -__builtin_inff();
    i = 0x7FFFFFFF;
  }
  __device__ __forceinline__ void push(float nv, int32_t ni) {
    if (better(nv, ni, v, i)) {
      v = nv;
      i = ni;
    }
  }
  // Push for ids that arrive in increasing order: a strict '>' already keeps
  // the smaller id on a tie.
  __device__ __forceinline__ void push_ascending(float nv, int32_t ni) {
    const bool gt = nv > v;
    v = gt ? nv : v;
    i = gt ? ni : i;
  }
  // Combine with the pair held by lane (lane ^ mask).
  __device__ __forceinline__ void xor_reduce(int mask) {
    const float ov = __shfl_xor(v, mask, kWave);
    const int32_t oi = __shfl_xor(i, mask, kWave);
    push(ov, oi);
  }
};

// Lane-strided argmax over P pairs (element p at o(p)), with the loads of
// kMergeUnroll strides issued before any comparison so that they are in
// flight together (the pairs were just written and sit in L2; one at a time
// they would cost one round trip each).  The comparator orders by value,
// then id, so the push order does not change the result.
constexpr int kMergeUnroll = 8;
template <class Off>
__device__ __forceinline__ void strided_argmax(const float* __restrict__ val,
                                               const int32_t* __restrict__ idx, int32_t P,
                                               int lane, Off o, ArgMax& m) {
  for (int p0 = lane; p0 < P; p0 += kWave * kMergeUnroll) {
    float v[kMergeUnroll];
    int32_t i[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int p = p0 + u * kWave;
      const bool in = p < P;
      v[u] = in ? val[o(p)] : -__builtin_inff();
      i[u] = in ? idx[o(p)] : 0x7FFFFFFF;
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) m.push(v[u], i[u]);
  }
}

// ---------------------------------------------------------------------------
// Running log-sum-exp, log sum_i exp(t_i), of a stream of scaled logits t_i,
// kept as (m, s) with m the running maximum and s = sum_i exp(t_i - m)
// (online normaliser: the maximum is folded in as it grows).  Masked
// entries are pushed as -FLT_MAX: finite, so no inf - inf arises, and their
// exponential underflows to 0 beside any real entry.  exp is the hardware
// exp2 of x log2(e).
// ---------------------------------------------------------------------------
struct LseAcc {
  float m, s;
  static constexpr float kMasked = -3.402823466e38f;
  __device__ __forceinline__ static float ex(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
  }
  __device__ __forceinline__ void init() {
    m = kMasked;
    s = 0.0f;
  }
  __device__ __forceinline__ void push4(f32x4 t) {
    const float nm = fmaxf(m, fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
    s = s * ex(m - nm) + ((ex(t[0] - nm) + ex(t[1] - nm)) + (ex(t[2] - nm) + ex(t[3] - nm)));
    m = nm;
  }
  __device__ __forceinline__ void merge(float om, float os) {
    const float nm = fmaxf(m, om);
    s = s * ex(m - nm) + os * ex(om - nm);
    m = nm;
  }
  __device__ __forceinline__ void xor_reduce(int mask) {
    const float om = __shfl_xor(m, mask, kWave);
    const float os = __shfl_xor(s, mask, kWave);
    merge(om, os);
  }
  // log-sum-exp; greedy rows report the maximum (their distribution's mode)
  __device__ __forceinline__ float value(bool greedy) const {
    return greedy ? m : m + __builtin_amdgcn_logf(s) * 0.693147180559945309f;
  }
};

// Row temperature -> (greedy flag, fp32 reciprocal).  Greedy when T is not a
// positive number (0, -0, negative, NaN): the T -> 0 limit of the sampler.
__device__ __forceinline__ bool row_is_greedy(float T) { return !(T > 0.0f); }

__device__ __forceinline__ float row_inv_temperature(float T) {
  return row_is_greedy(T) ? 1.0f : __fdiv_rn(1.0f, T);
}


// Pushes the scores of four consecutive logits z (local vocabulary rows
// v0 .. v0+3, global ids gv0 .. gv0+3 with gv0 % 4 == 0, batch row `row`)
// into `best`; the four ids share one Philox block.  Rows outside [0, V)
// score -inf and never win; greedy rows score the logit itself.  Everything
// is computed on every lane and selected, without branches: the lanes of a
// wave hold different batch rows, so a branch would serialise.  With LSE,
// also folds the scaled logits z / T (greedy rows: z) of the valid rows into
// `lse`.
template <bool LSE = false>
__device__ __forceinline__ void push_four(ArgMax& best, f32x4 z, int v0, int32_t V, uint32_t gv0,
                                          uint32_t row, uint64_t step, bool greedy,
                                          float inv_t, const Philox& philox,
                                          LseAcc* lse = nullptr) {
  const u32x4 w = philox(noise_counter(gv0, row, step));
  f32x4 t;
  static_for<4>([&](auto rc) FS_INLINE {
    constexpr int r = decltype(rc)::value;
    const float scaled = __fmul_rn(z[r], inv_t);
    const float noisy = __fadd_rn(scaled, gumbel_from_bits(w[r]));
    const bool valid = static_cast<uint32_t>(v0 + r) < static_cast<uint32_t>(V);
    float s = greedy ? z[r] : noisy;
    s = valid ? s : -__builtin_inff();
    best.push_ascending(s, static_cast<int32_t>(gv0 + r));
    if (LSE) t[r] = valid ? (greedy ? z[r] : scaled) : LseAcc::kMasked;
  });
  if (LSE) lse->push4(t);
}

}  // namespace fs
