// fs_pack.hip -- W in fragment order for the packed samplers.
//
// The samplers' main loops read W one MFMA A-fragment at a time: 16 rows x 32
// k, each lane 16 bytes.  From a row-major [V][D] W such a load takes 64 bytes
// from each of 16 rows 8 KB apart, and a tile's k-steps revisit every row many
// microseconds apart, which costs HBM page locality.  The packed layout
// (packed_frag in fs_mma.hpp) stores each 16-row group of the sampler's grid
// k-step by k-step as the 64 lanes' pieces, so a fragment is 1 KB contiguous
// and a group is streamed front to back.  The fragments' contents are those of
// the row-major path, so results are identical.
#include "fs_device.hpp"
#include "fs_internal.hpp"

namespace fs {

namespace {

// One thread per 16-byte piece of the packed output (writes are contiguous).
__global__ __launch_bounds__(256) void pack_weights_kernel(const __bf16* __restrict__ W,
                                                           int32_t V, int32_t D, int32_t shift,
                                                           int64_t pieces,
                                                           __bf16* __restrict__ Wp) {
  const int64_t ksteps = D / 32;
  for (int64_t p = blockIdx.x * 256ll + threadIdx.x; p < pieces; p += 256ll * gridDim.x) {
    const int lane = static_cast<int>(p & (kWave - 1));
    const int64_t gs = p >> 6;
    const int64_t s = gs % ksteps, g = gs / ksteps;
    const int64_t v = g * 16 + (lane & 15) - shift;
    const int64_t k = s * 32 + 8 * (lane >> 4);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (v >= 0 && v < V) x = *reinterpret_cast<const u32x4*>(W + v * D + k);
    *reinterpret_cast<u32x4*>(Wp + p * 8) = x;
  }
}

}  // namespace

hipError_t launch_pack_weights(const __bf16* W, int32_t V, int32_t D, int32_t vocab_offset,
                               __bf16* Wp, hipStream_t stream) {
  const int64_t pieces = packed_groups(V, vocab_offset) * (D / 32) * kWave;
  const int64_t blocks = (pieces + 255) / 256;
  pack_weights_kernel<<<dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)), 256, 0,
                        stream>>>(W, V, D, vocab_offset & 3, pieces, Wp);
  return hipGetLastError();
}

}  // namespace fs
