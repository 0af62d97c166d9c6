// fs_internal.hpp -- host-side interface between the C ABI (fs_api.hip) and
// the kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fs {

// Most vocabulary groups one grouped launch takes (fs_sample_groups_lse).
constexpr int kMaxGroups = 64;

struct SampleArgs {
  const __bf16* h;
  const __bf16* W;
  int32_t B, D, V, vocab_offset;
  const float* temperature;
  uint64_t seed, step;
  float* part_val;    // [B][S] per-block partial maxima
  int32_t* part_idx;  // [B][S] their global ids
  float* part_lse;    // [B][S] per-block log-sum-exp of z / T (grouped sampler), or null
  int32_t S;          // number of vocabulary blocks (set by the launcher)
  // If non-null and *live == 0 when a block starts, the block does nothing
  // (the online sampler's later chunks, once every row is final).
  const int32_t* live = nullptr;
  // W in fragment order (fs_pack_weights) instead of row-major [V][D]
  bool w_packed = false;
  // Vocabulary groups of one grouped launch: group g holds W rows
  // [grp_rows[g], grp_rows[g+1]) and vocabulary blocks [grp_tiles[g],
  // grp_tiles[g+1]).  Each group's block grid starts at its own first row
  // (shifted down to a global id divisible by 4), so no block holds rows of
  // two groups.  n_groups == 0: one slice, the whole of W.  The launcher fills
  // grp_tiles from grp_rows, and grp_span: group g's partials are entries
  // [grp_tiles[g], grp_tiles[g+1]) of each row, or with grp_span > 0 (the
  // persistent kernels, whose blocks sweep a group's 16-row groups) entries
  // [grp_tiles[g], min(grp_tiles[g+1], grp_tiles[g] + grp_span)).
  int32_t n_groups = 0;
  int32_t grp_rows[kMaxGroups + 1];
  int32_t grp_tiles[kMaxGroups + 1];
  int32_t grp_span = 0;
};

// One fused-sampler configuration (a main-loop policy and its tile shape).
struct FusedConfig {
  const char* name;
  int rows_per_block;
  hipError_t (*launch)(SampleArgs&, hipStream_t);
  bool (*supports)(int32_t B, int32_t D);
  int order;  // configurations of equal order sum the contraction identically
  bool packed_w;  // can read W in fragment order
};

// Configuration lists of the translation units fs_configs_*.hip.
int fused_configs_small(const FusedConfig** out);
int fused_configs_lds(const FusedConfig** out);
int fused_configs_dma_a(const FusedConfig** out);
int fused_configs_dma_b(const FusedConfig** out);
int fused_configs_dma_ntl(const FusedConfig** out);

// ---- fused sampler (fs_fused.hip) ----
int num_fused_configs();
const char* fused_config_name(int id);
int fused_rows_per_block(int id);
// Automatic choice; `packed`: for W in fragment order (fs_pack_weights);
int fused_auto_config(int32_t B, int32_t D, int32_t V, bool packed = false);
bool fused_config_supports(int id, int32_t B, int32_t D);
bool fused_config_reads_packed(int id);
// Configurations with equal order sum each logit's products identically.
int fused_config_order(int id);
// Smallest rows-per-block over all configurations: bounds the split count.
constexpr int kMinRowsPerBlock = 16;
// Launch configuration `id`; sets a.S to the number of vocabulary blocks.
hipError_t launch_fused(int id, SampleArgs& a, hipStream_t stream);

// Per-row argmax over P partials; element (p, b) at p * stride_p + b * stride_b.
hipError_t launch_merge(const float* val, const int32_t* idx, int32_t P, int32_t B,
                        int64_t stride_p, int64_t stride_b, int32_t* out_ids,
                        float* out_val, hipStream_t stream);

// Per-row argmax and log-sum-exp over the S tile partials of one slice
// (element (b, t) at b * S + t).
hipError_t launch_merge_tiles_lse(const float* val, const int32_t* idx, const float* lse,
                                  int32_t S, int32_t B, const float* temperature,
                                  int32_t* out_ids, float* out_val, float* out_lse,
                                  hipStream_t stream);
// Per-group argmax and log-sum-exp of a grouped launch's tile partials
// (element (b, t) at b * S + t; group g holds tiles [grp_tiles[g],
// grp_tiles[g+1])) into slot g of G x B part-major outputs.
// Group g's partials in each row: entries [t[g], end[g]).
struct GroupTiles {
  int32_t n;
  int32_t t[kMaxGroups + 1];
  int32_t end[kMaxGroups];
};
hipError_t launch_merge_group_tiles_lse(const float* val, const int32_t* idx, const float* lse,
                                        int32_t S, int32_t B, const GroupTiles& groups,
                                        const float* temperature, float* out_val,
                                        int32_t* out_idx, float* out_lse, hipStream_t stream);
// Grouped merge over P group partials, part-major (element (p, b) at p * B + b).
hipError_t launch_merge_groups_lse(const float* val, const int32_t* idx, const float* lse,
                                   int32_t P, int32_t B, const float* temperature,
                                   uint64_t seed, uint64_t step, int32_t* out_ids,
                                   float* out_val, float* out_lse, hipStream_t stream);

// ---- online sampler with early finalisation (fs_online.hip) ----
// Euclidean norm of each of the n rows of X (bf16, row length D), fp64.
hipError_t launch_row_norms(const __bf16* X, int32_t n, int32_t D, double* out,
                            hipStream_t stream);
// The same from fragment-order W (packed for vocab_offset mod 4).
hipError_t launch_packed_row_norms(const __bf16* Wp, int32_t V, int32_t D, int32_t vocab_offset,
                                   double* out, hipStream_t stream);
// out[0] = max of x[0 .. n).
hipError_t launch_max_reduce(const double* x, int32_t n, double* out, hipStream_t stream);
// later[c] = max(chunk_max[c+1 .. n_chunks)), later[n_chunks - 1] = 0.
hipError_t launch_suffix_max(const double* chunk_max, int32_t n_chunks, double* later,
                             hipStream_t stream);
// Row norms of h, running pairs (-inf, INT32_MAX), done flags and live counts cleared.
hipError_t launch_online_init(const __bf16* h, int32_t B, int32_t D, int32_t n_chunks,
                              double* hnorm, int32_t* done, int32_t* live, int32_t* out_ids,
                              float* out_val, int32_t* out_chunks, hipStream_t stream);
// Chunk c of the online sampler: merges the chunk's S tile partials into the
// running pair of every row not yet final, tests the bound and counts the
// rows still live into live[c].  Does nothing if c > 0 and live[c-1] == 0.
hipError_t launch_online_step(const float* part_val, const int32_t* part_idx, int32_t S,
                              int32_t B, int32_t c, int32_t n_chunks, const double* later,
                              const double* hnorm, const float* temperature, double g_max,
                              double margin, int32_t* done, int32_t* live, int32_t* out_ids,
                              float* out_val, int32_t* out_chunks, hipStream_t stream);

// ---- fragment-order W (fs_pack.hip) ----
// Groups of 16 rows of the grid shifted by vocab_offset mod 4.
inline int64_t packed_groups(int32_t V, int32_t vocab_offset) {
  return (static_cast<int64_t>(V) + (vocab_offset & 3) + 15) / 16;
}
hipError_t launch_pack_weights(const __bf16* W, int32_t V, int32_t D, int32_t vocab_offset,
                               __bf16* Wp, hipStream_t stream);

hipError_t launch_debug_noise(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0,
                              int64_t n, uint32_t* bits, float* g, hipStream_t stream);
hipError_t launch_debug_gumbel(const uint32_t* bits, int64_t n, float* g,
                               hipStream_t stream);

// ---- unfused baseline (fs_unfused.hip) ----
size_t unfused_workspace_bytes(int32_t B, int32_t V);
hipError_t launch_unfused(const SampleArgs& a, int32_t* out_ids, float* out_val,
                          void* workspace, hipStream_t stream);

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace fs
