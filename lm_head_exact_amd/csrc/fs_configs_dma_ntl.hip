// fs_configs_dma_ntl.hip -- DMA-staged configurations with non-temporal W
// loads: the twins (name + "_ntl1") the packed-W choice takes (one of several
// translation units, compiled in parallel).
#include "fs_sampler.hpp"

namespace fs {

int fused_configs_dma_ntl(const FusedConfig** out) {
  static const FusedConfig k[] = {
      FS_DMAN(2, 16, 8, 64, 4, 4, 4, 2),
      FS_DMAN(4, 4, 8, 64, 4, 3, 4, 2),
      FS_DMAN(4, 8, 8, 64, 4, 3, 4, 2),
      FS_DMAN(5, 4, 8, 64, 4, 3, 4, 2),
      FS_DMAN(5, 8, 8, 64, 2, 3, 4, 2),
      FS_DMAN(1, 4, 4, 64, 8, 3, 4, 2),
      FS_DMAN(1, 8, 4, 64, 8, 3, 4, 2),
      FS_DMAPN(2, 16, 8, 64, 4, 4, 4, 2),
      FS_DMAPN(1, 8, 8, 128, 8, 3, 4, 2),
  };
  *out = k;
  return static_cast<int>(sizeof(k) / sizeof(k[0]));
}

}  // namespace fs
