// fs_configs_lds.hip -- LDS-staged configurations of the fused sampler
// (one of several translation units, compiled in parallel).
#include "fs_sampler.hpp"

namespace fs {

int fused_configs_lds(const FusedConfig** out) {
  static const FusedConfig k[] = {
      FS_LDS(2, 4, 4, 64, 4, 0),        // B <= 64 when the DMA grid would leave CUs idle
      FS_LDSR(4, 8, 4, 64, 4, 1, 4),    // B <= 128, likewise
      FS_LDSR(2, 16, 4, 64, 4, 1, 4),   // B > 128, likewise
      FS_LDSR(2, 8, 4, 64, 8, 1, 4),
  };
  *out = k;
  return static_cast<int>(sizeof(k) / sizeof(k[0]));
}

}  // namespace fs
