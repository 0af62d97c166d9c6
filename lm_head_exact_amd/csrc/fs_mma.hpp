// fs_mma.hpp -- the LM-head contraction tile on gfx950 bf16 MFMA.
//
// One wavefront computes a (MR*16 vocab rows) x (NT*16 batch rows) block of
// logits z[b][v] = sum_d h[b][d] W[v][d] with v_mfma_f32_16x16x32_bf16:
// W plays the MFMA "A" operand (rows = vocabulary), h the "B" operand
// (columns = batch).  Operand fragments are read straight from global memory
// into registers: every W element is used by exactly one wave, so staging W
// through LDS would only add traffic; h is small and stays in L1/L2.
//
// Register layouts (wave64, 16x16x32 bf16):
//   A fragment, lane l: row (l % 16), 8 consecutive k at 8 * (l / 16)
//   B fragment, lane l: col (l % 16), the same 8 k
//   C tile,     lane l: col (l % 16), rows 4 * (l / 16) + {0,1,2,3}
// A lane therefore loads 16 contiguous bytes of one W row per 32-wide k step,
// and each lane ends up holding four consecutive vocabulary rows of one batch
// row: exactly the four ids one Philox block covers.
#pragma once

#include "fs_device.hpp"

namespace fs {

__device__ __forceinline__ bf16x8 load_frag(const __bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_frag() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Accumulate the whole K = D contraction for one wave's block.
//   W      [V][D] bf16, h [B][D] bf16
//   row0   first vocabulary row of the block; rows >= V are clamped to V-1
//          (their results are discarded by the caller)
//   col0   first batch row; columns >= B read zeros
template <int MR, int NT>
__device__ __forceinline__ void mma_block(const __bf16* __restrict__ W,
                                          const __bf16* __restrict__ h, int32_t B,
                                          int32_t D, int32_t V, int32_t row0, int32_t col0,
                                          f32x4 (&acc)[MR][NT]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int li = lane & 15, kb = lane >> 4;

  const __bf16* arow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int v = min(row0 + m * 16 + li, V - 1);
    arow[m] = W + static_cast<size_t>(v) * D + 8 * kb;
  }
  const __bf16* brow[NT];
  bool bvalid[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int b = col0 + n * 16 + li;
    bvalid[n] = b < B;
    brow[n] = h + static_cast<size_t>(min(b, B - 1)) * D + 8 * kb;
  }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = D >> 5;
#pragma unroll 4
  for (int t = 0; t < ksteps; ++t) {
    bf16x8 af[MR], bfr[NT];
#pragma unroll
    for (int m = 0; m < MR; ++m) af[m] = load_frag(arow[m] + t * 32);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 x = load_frag(brow[n] + t * 32);
      bfr[n] = bvalid[n] ? x : zero_frag();
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
  }
  if (D & 31) {  // last partial step: D % 8 == 0, so a lane's 8 k are all in or all out
    const int k = ksteps * 32 + 8 * kb;
    const bool kin = k < D;
    bf16x8 af[MR], bfr[NT];
#pragma unroll
    for (int m = 0; m < MR; ++m) af[m] = kin ? load_frag(arow[m] + ksteps * 32) : zero_frag();
#pragma unroll
    for (int n = 0; n < NT; ++n)
      bfr[n] = (kin && bvalid[n]) ? load_frag(brow[n] + ksteps * 32) : zero_frag();
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
  }
}

}  // namespace fs
