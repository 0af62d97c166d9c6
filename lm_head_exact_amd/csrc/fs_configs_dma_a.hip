// fs_configs_dma_a.hip -- DMA-staged configurations of the fused sampler chosen automatically
// (one of several translation units, compiled in parallel).
#include "fs_sampler.hpp"

namespace fs {

int fused_configs_dma_a(const FusedConfig** out) {
  static const FusedConfig k[] = {
      FS_DMAG(4, 4, 8, 64, 4, 3, 4, 2),   // B <= 64
      FS_DMAG(4, 8, 8, 64, 4, 3, 4, 2),   // B <= 128
      FS_DMAG(2, 16, 8, 64, 4, 4, 4, 2),  // B > 128 (batch blocks of 256)
      FS_DMAG(2, 16, 8, 128, 4, 2, 4, 2),
      FS_DMAP(2, 16, 8, 128, 4, 2, 4, 2), // B > 256 (several batch blocks)
      FS_DMAP(1, 8, 8, 128, 8, 3, 4, 2),  // short vocabularies, B > 128
  };
  *out = k;
  return static_cast<int>(sizeof(k) / sizeof(k[0]));
}

}  // namespace fs
