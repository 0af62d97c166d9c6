// fs_configs_dma_b.hip -- further DMA-staged configurations of the fused sampler: the taller
// and narrower blocks the automatic choice takes, and (only in a build with FS_TUNING_SWEEPS
// defined) the alternatives kept for tuning sweeps (one of several translation units, compiled
// in parallel).
#include "fs_sampler.hpp"

namespace fs {

int fused_configs_dma_b(const FusedConfig** out) {
  static const FusedConfig k[] = {
      FS_DMAG(5, 4, 8, 64, 4, 3, 4, 2),   // B <= 64, 640-row blocks
      FS_DMAG(5, 8, 8, 64, 2, 3, 4, 2),   // B <= 128, 640-row blocks
      FS_DMAG(1, 4, 4, 64, 8, 3, 4, 2),   // short vocabularies: 64-row blocks
      FS_DMAG(1, 8, 4, 64, 8, 3, 4, 2),
#ifdef FS_TUNING_SWEEPS
      FS_DMA(2, 16, 8, 64, 4, 4, 4),
      FS_DMA(4, 8, 8, 64, 4, 3, 4),
      FS_DMAG(2, 16, 8, 64, 8, 3, 4, 2),
      FS_DMAG(2, 8, 8, 64, 4, 4, 4, 2),
      FS_DMAR(2, 16, 8, 64, 4, 4, 4, 2),  // block-rotated chunk order
      FS_DMAR(4, 8, 8, 64, 4, 3, 4, 2),
      FS_DMAR(4, 4, 8, 64, 4, 3, 4, 2),
      FS_DMAW(8, 4, 8, 64, 2, 3, 4, 2, 2),  // two batch groups of waves (WB = 2)
#endif
  };
  *out = k;
  return static_cast<int>(sizeof(k) / sizeof(k[0]));
}

}  // namespace fs
