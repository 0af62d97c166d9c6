// fs_configs_small.hip -- persistent K-split, K-split and streaming configurations of the fused sampler
// (one of several translation units, compiled in parallel).
#include "fs_sampler.hpp"

namespace fs {

int fused_configs_small(const FusedConfig** out) {
  static const FusedConfig k[] = {
      FS_PERSIST(1, 8, 16, 8),   // D = 4096, B <= 16
      FS_PERSIST(2, 8, 16, 8),   // D = 4096, B <= 32
      FS_PERSIST(1, 8, 32, 8),   // D = 8192, B <= 16
      FS_KSPLIT(1, 1, 4, 8, 0),  // B <= 8 when no persistent shape fits
      FS_STREAM(4, 1, 4, 4, 0),  // any D: fallback for B <= 16
      FS_STREAM(2, 4, 4, 4, 0),  // any D: fallback for larger B
      FS_PERSISTN(1, 8, 32, 8),   // packed W, D = 8192, B <= 16
      FS_PERSISTN(2, 8, 16, 4),   // packed W, B <= 32
      FS_PERSISTN(1, 16, 8, 4),   // packed W, B <= 16
  };
  *out = k;
  return static_cast<int>(sizeof(k) / sizeof(k[0]));
}

}  // namespace fs
