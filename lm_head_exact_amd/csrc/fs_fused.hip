// fs_fused.hip -- the fused sampler's configuration table and automatic
// choice, the merge kernels (tile partials, shard partials, grouped
// partials) and the noise diagnostics.  The sampler kernels themselves are
// in fs_sampler.hpp, instantiated by fs_configs_*.hip.
#include <atomic>
#include <cstring>
#include <string>
#include <vector>

#include "fs_device.hpp"
#include "fs_internal.hpp"

namespace fs {

// One wave per batch row: argmax over P (value, id) pairs.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ val,
                                                    const int32_t* __restrict__ idx,
                                                    int32_t P, int32_t B, int64_t stride_p,
                                                    int64_t stride_b, int32_t* out_ids,
                                                    float* out_val) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wave
  ArgMax m;
  m.init();
  strided_argmax(val, idx, P, lane,
                 [&](int p) FS_INLINE { return p * stride_p + b * stride_b; }, m);
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) m.xor_reduce(mask);
  if (lane == 0) {
    out_ids[b] = m.i;
    out_val[b] = m.v;
  }
}

// One wave per batch row over its S tile partials (element (b, t) at
// b * S + t): the argmax as merge_kernel, and the log-sum-exp of the tiles'
// log-sum-exps (greedy rows: their maximum).
__global__ __launch_bounds__(256) void merge_tiles_lse_kernel(
    const float* __restrict__ val, const int32_t* __restrict__ idx, const float* __restrict__ lse,
    int32_t S, int32_t B, const float* __restrict__ temperature, int32_t* out_ids, float* out_val,
    float* out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wave
  ArgMax m;
  m.init();
  LseAcc l;
  l.init();
  for (int t = lane; t < S; t += kWave) {
    const int64_t o = static_cast<int64_t>(b) * S + t;
    m.push(val[o], idx[o]);
    l.merge(lse[o], 1.0f);  // a tile's log-sum-exp L is the pair (L, 1)
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    m.xor_reduce(mask);
    l.xor_reduce(mask);
  }
  if (lane == 0) {
    out_ids[b] = m.i;
    out_val[b] = m.v;
    out_lse[b] = l.value(row_is_greedy(temperature[b]));
  }
}

// Grouped launch: one wave per (batch row, group) over the group's partials
// (element (b, t) at b * S + t, group g's entries [groups.t[g],
// groups.end[g])), the argmax and log-sum-exp as merge_tiles_lse_kernel,
// into slot g of the G x B part-major outputs.
__global__ __launch_bounds__(256) void merge_group_tiles_lse_kernel(
    const float* __restrict__ val, const int32_t* __restrict__ idx, const float* __restrict__ lse,
    int32_t S, int32_t B, GroupTiles groups, const float* __restrict__ temperature,
    float* out_val, int32_t* out_idx, float* out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (b >= B) return;  // uniform per wave
  // the group's tile range, read with constant indices only (see the fused kernel)
  int t0 = 0, t1 = 0;
#pragma unroll
  for (int k = 0; k < kMaxGroups; ++k) {
    if (k == g) {
      t0 = groups.t[k];
      t1 = groups.end[k];
    }
  }
  ArgMax m;
  m.init();
  LseAcc l;
  l.init();
  for (int t = t0 + lane; t < t1; t += kWave) {
    const int64_t o = static_cast<int64_t>(b) * S + t;
    m.push(val[o], idx[o]);
    l.merge(lse[o], 1.0f);  // a tile's log-sum-exp L is the pair (L, 1)
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    m.xor_reduce(mask);
    l.xor_reduce(mask);
  }
  if (lane == 0) {
    const int64_t o = static_cast<int64_t>(g) * B + b;
    out_val[o] = m.v;
    out_idx[o] = m.i;
    out_lse[o] = l.value(row_is_greedy(temperature[b]));
  }
}

// Grouped merge, one wave per batch row over P group partials (part-major,
// element (p, b) at p * B + b).  The categorical distribution factorises as
// P(i) = P(G) P(i | G) with P(G) proportional to exp(LSE_G): each group's
// partial already holds a sample of P(i | G), so the row takes group
// argmax_p (lse_p + gamma_p), gamma_p a Gumbel draw independent of the token
// noise (counter word 0 = 2^31 | p, which token counters, gv / 4 < 2^29,
// never reach), ties to the smaller p; greedy rows take argmax_p lse_p.  It
// also returns the row's total log-sum-exp over the groups.
__global__ __launch_bounds__(256) void merge_groups_lse_kernel(
    const float* __restrict__ val, const int32_t* __restrict__ idx, const float* __restrict__ lse,
    int32_t P, int32_t B, const float* __restrict__ temperature, uint64_t seed, uint64_t step,
    int32_t* out_ids, float* out_val, float* out_lse) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;  // uniform per wave
  const bool greedy = row_is_greedy(temperature[b]);
  const Philox philox(seed);
  ArgMax m;  // (key, group) with ties to the smaller group
  m.init();
  LseAcc l;
  l.init();
  for (int p = lane; p < P; p += kWave) {
    const float lp = lse[static_cast<int64_t>(p) * B + b];
    float key = lp;
    if (!greedy) {
      const u32x4 w = philox(u32x4{0x80000000u | static_cast<uint32_t>(p), static_cast<uint32_t>(b),
                                   static_cast<uint32_t>(step), static_cast<uint32_t>(step >> 32)});
      key = __fadd_rn(lp, gumbel_from_bits(w.x));
    }
    m.push(key, p);
    l.merge(lp, 1.0f);
  }
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    m.xor_reduce(mask);
    l.xor_reduce(mask);
  }
  if (lane == 0) {
    // m.i < P unless every key is NaN (NaN inputs are undefined behaviour);
    // clamp so that even then the read stays inside the partials
    const int p_star = m.i >= 0 && m.i < P ? m.i : 0;
    const int64_t o = static_cast<int64_t>(p_star) * B + b;
    out_ids[b] = idx[o];
    out_val[b] = val[o];
    out_lse[b] = l.value(greedy);
  }
}

__global__ __launch_bounds__(256) void debug_noise_kernel(uint64_t seed, uint64_t step,
                                                          uint32_t row, uint32_t gv0,
                                                          int64_t n, uint32_t* bits,
                                                          float* g) {
  const Philox philox(seed);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const uint32_t gv = gv0 + static_cast<uint32_t>(i);
    const uint32_t x = pick_word(philox(noise_counter(gv, row, step)), gv & 3u);
    if (bits) bits[i] = x;
    if (g) g[i] = gumbel_from_bits(x);
  }
}

__global__ __launch_bounds__(256) void debug_gumbel_kernel(const uint32_t* bits, int64_t n,
                                                           float* g) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x)
    g[i] = gumbel_from_bits(bits[i]);
}

// ---------------------------------------------------------------------------
// Host side: configuration table and launchers.
// ---------------------------------------------------------------------------
namespace {

// All configurations, in the order of the translation units' lists.
const std::vector<FusedConfig>& configs() {
  static const std::vector<FusedConfig> all = [] {
    std::vector<FusedConfig> v;
    for (auto part : {&fused_configs_small, &fused_configs_lds, &fused_configs_dma_a,
                      &fused_configs_dma_b, &fused_configs_dma_ntl}) {
      const FusedConfig* k = nullptr;
      const int n = part(&k);
      v.insert(v.end(), k, k + n);
    }
    return v;
  }();
  return all;
}

int config_id(const char* name) {
  const auto& c = configs();
  for (size_t i = 0; i < c.size(); ++i)
    if (std::strcmp(c[i].name, name) == 0) return static_cast<int>(i);
  return -1;
}

}  // namespace

int num_fused_configs() { return static_cast<int>(configs().size()); }

const char* fused_config_name(int id) {
  return (id >= 0 && id < num_fused_configs()) ? configs()[id].name : nullptr;
}

int fused_rows_per_block(int id) {
  return (id >= 0 && id < num_fused_configs()) ? configs()[id].rows_per_block : 0;
}

int fused_config_order(int id) {
  return (id >= 0 && id < num_fused_configs()) ? configs()[id].order : -1;
}

bool fused_config_reads_packed(int id) {
  return id >= 0 && id < num_fused_configs() && configs()[id].packed_w;
}


bool fused_config_supports(int id, int32_t B, int32_t D) {
  return id >= 0 && id < num_fused_configs() && configs()[id].supports(B, D);
}

namespace {
// CU count of the current device, cached per device (0 until known; callers
// on several threads may race to fill an entry, with the same value).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const int known = cached[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (cacheable) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Share of CU slots busy over the whole grid of a configuration that runs one
// block per CU: blocks / (rounds * CUs).  A grid whose last round is mostly
// empty wastes that round.
double one_per_cu_fill(int id, int32_t V) {
  const int cus = device_cus();
  if (cus <= 0) return 0.0;
  const int rows = fused_rows_per_block(id);
  const long blocks = (static_cast<long>(V) + rows - 1) / rows;
  const long rounds = (blocks + cus - 1) / cus;
  return static_cast<double>(blocks) / (static_cast<double>(rounds) * cus);
}
}  // namespace

static int auto_config_shape(int32_t B, int32_t D, int32_t V, bool packed);

// The configuration with the same loop and tile shape but non-temporal W
// loads (name + "_ntl1"), if there is one, else `id`.  On fragment-order W
// each wave streams contiguous memory that is read exactly once, and the
// non-temporal hint then raises the rate (Llama-3 head: 172 -> 158 us at
// B = 1, 182 -> 163 us at B = 64, 269 -> 252 us at B = 256); on row-major W
// it lowers it, so only the packed choice takes these twins.
static int non_temporal_twin(int id) {
  static const std::vector<int> twin = [] {
    std::vector<int> t(configs().size());
    for (size_t i = 0; i < t.size(); ++i) {
      const int j = config_id((std::string(configs()[i].name) + "_ntl1").c_str());
      t[i] = j >= 0 && configs()[j].packed_w ? j : static_cast<int>(i);
    }
    return t;
  }();
  return id >= 0 && id < static_cast<int>(twin.size()) ? twin[id] : id;
}

int fused_auto_config(int32_t B, int32_t D, int32_t V, bool packed) {
  const int id = auto_config_shape(B, D, V, packed);
  return packed ? non_temporal_twin(id) : id;
}

static int auto_config_shape(int32_t B, int32_t D, int32_t V, bool packed) {
  static const int persist[] = {config_id("persist_nt1_nw8_ks16_p8"),
                                config_id("persist_nt2_nw8_ks16_p8"),
                                config_id("persist_nt1_nw8_ks32_p8")};
  // on packed W (non-temporal loads) the block shape and load ring depth
  // that time best per batch tile (Llama-3 head: B = 1 156 us with 16 waves
  // of 8 k-steps and a 4-step ring, against 159 us with 8 waves and 16 steps
  // and 159 with 8 and 8; B = 32 162.5 against 166.7 us with a 4-step ring)
  static const int persist_packed[] = {config_id("persist_nt1_nw16_ks8_p4_ntl1"),
                                       config_id("persist_nt2_nw8_ks16_p4_ntl1"),
                                       config_id("persist_nt1_nw8_ks32_p8_ntl1")};
  static const int ksplit = config_id("ksplit_mr1_nt1_nw4_p8_ntl0");
  // batch-tiled loops: the DMA-staged loop (one 8-wave block per CU) when its
  // grid fills the CUs; for a short vocabulary the same loop on 64-row blocks
  // of four waves; else the LDS loop (smaller blocks, two per CU)
  static const int dma64 = config_id("dma_mr4_nt4_nw8_kc64_p4_s3_br4_g2");
  static const int dma64_tall = config_id("dma_mr5_nt4_nw8_kc64_p4_s3_br4_g2");
  static const int dma128 = config_id("dma_mr4_nt8_nw8_kc64_p4_s3_br4_g2");
  static const int dma128_tall = config_id("dma_mr5_nt8_nw8_kc64_p2_s3_br4_g2");
  static const int dma256 = config_id("dma_mr2_nt16_nw8_kc64_p4_s4_br4_g2");
  static const int dma256_kc128 = config_id("dma_mr2_nt16_nw8_kc128_p4_s2_br4_g2");
  static const int dma_paired = config_id("dmapair_mr2_nt16_nw8_kc128_p4_s2_br4_g2");
  // (packed W only: named by its non-temporal form, the one the packed choice takes)
  static const int dma_paired_kc64 = config_id("dmapair_mr2_nt16_nw8_kc64_p4_s4_br4_g2_ntl1");
  static const int dma64_short = config_id("dma_mr1_nt4_nw4_kc64_p8_s3_br4_g2");
  static const int dma128_short = config_id("dma_mr1_nt8_nw4_kc64_p8_s3_br4_g2");
  // above 128 batch rows on a short vocabulary: 128-row blocks of 128 batch
  // rows on the paired grid, so that each block stages half as much of h (a
  // vocabulary shard at B = 256, D = 8192 stages 4 MB of h per 64-row block,
  // 1.07 GB from L2 per step against 0.26 GB of W; 83 against 97 us)
  static const int dma_paired_short = config_id("dmapair_mr1_nt8_nw8_kc128_p8_s3_br4_g2");
  static const int lds64 = config_id("lds_mr2_nt4_nw4_kc64_p4_ntl0");
  static const int lds128 = config_id("lds_mr4_nt8_nw4_kc64_p4_wb1_br4");
  static const int lds256 = config_id("lds_mr2_nt16_nw4_kc64_p4_wb1_br4");
  static const int lds_narrow = config_id("lds_mr2_nt8_nw4_kc64_p8_wb1_br4");
  static const int stream_small = config_id("stream_mr4_nt1_nw4_p4_ntl0");
  static const int stream_big = config_id("stream_mr2_nt4_nw4_p4_ntl0");
  for (int id : packed ? persist_packed : persist)
    if (fused_config_supports(id, B, D)) return id;
  // (the K-split loop reads row-major W only: packed W goes on to the DMA loop)
  if (!packed && B <= 8 && fused_config_supports(ksplit, B, D)) return ksplit;
  // DMA candidates per batch width, first choice first: 512-row blocks, else
  // 640-row blocks where those fill the CUs better (a vocabulary of ~152k
  // rows gives 297 blocks of 512, two rounds on 256 CUs, but 238 of 640).
  // At 256 batch rows, rows longer than 4096 run faster with 128-wide staged
  // chunks (2-3% in sweeps at D = 5120 and 8192; equal at 4096).  Above 256
  // batch rows the batch blocks of one vocabulary tile run side by side on
  // one XCD and share its W rows through L2 (9-12% at B = 384 and 512 at
  // D = 4096, 5120 and 8192).
  //
  // Every candidate sums each logit's products in k order in one wave, like
  // the LDS loops below: the choice may depend on V, so a vocabulary shard
  // gets the same bits as the same rows inside a whole-vocabulary call.
  //
  // On fragment-order (packed) W the 640-row blocks come first up to 128
  // batch rows whenever they fill the CUs (Llama-3 head, non-temporal twins:
  // 163 against 194 us at B = 64, 175 against 194 us at B = 128): each wave
  // then streams five contiguous 16-row groups.  At 256 batch rows the
  // 64-wide staged chunks win at every D there (431 against 437 us on the
  // Qwen3 head, 502 against 510 us at D = 8192), and on the paired grid above
  // 256 batch rows (B = 512: 873 against 917 us at D = 8192, 483 against 500
  // us on the Llama-3 head, 681 against 708 us on the Qwen3 head).
  struct Pick { int dma[2]; int dma_short; int lds; };
  const int dma256_first = D <= 4096 ? dma256 : dma256_kc128;
  const Pick p = B <= 64    ? (packed ? Pick{{dma64_tall, dma64}, dma64_short, lds64}
                                      : Pick{{dma64, dma64_tall}, dma64_short, lds64})
                 : B <= 128 ? (packed ? Pick{{dma128_tall, dma128}, dma128_short, lds128}
                                      : Pick{{dma128, dma128_tall}, dma128_short, lds128})
                 : B <= 256 ? (packed ? Pick{{dma256, dma256_kc128}, dma_paired_short, lds256}
                                      : Pick{{dma256_first, dma256}, dma_paired_short, lds256})
                 : packed   ? Pick{{dma_paired_kc64, dma256}, dma_paired_short, lds256}
                            : Pick{{dma_paired, dma256_first}, dma_paired_short, lds256};
  // below three quarters of the CUs busy on average over the rounds the LDS
  // loop's smaller blocks win (sweeps: 0.58 loses by 15-30%, 0.77 wins by 2-5%)
  constexpr double kMinFill = 0.75;
  for (int id : p.dma)
    if (fused_config_supports(id, B, D) && one_per_cu_fill(id, V) >= kMinFill) return id;
  // a short vocabulary (one shard of a split head) leaves CUs idle even under
  // the LDS loop's blocks: 64-row blocks of four waves fill them and still
  // read each W row once per batch block
  const int cus = device_cus();
  const bool short_v = cus > 0 && (static_cast<long>(V) + fused_rows_per_block(p.lds) - 1) /
                                          fused_rows_per_block(p.lds) < static_cast<long>(cus);
  if (short_v && fused_config_supports(p.dma_short, B, D)) return p.dma_short;
  if (short_v && B > 128 && fused_config_supports(lds_narrow, B, D)) return lds_narrow;
  if (fused_config_supports(p.lds, B, D)) return p.lds;
  return B <= 16 ? stream_small : stream_big;
}

hipError_t launch_fused(int id, SampleArgs& a, hipStream_t stream) {
  return configs()[id].launch(a, stream);
}

hipError_t launch_merge(const float* val, const int32_t* idx, int32_t P, int32_t B,
                        int64_t stride_p, int64_t stride_b, int32_t* out_ids,
                        float* out_val, hipStream_t stream) {
  const dim3 grid((B + 3) / 4);
  merge_kernel<<<grid, 256, 0, stream>>>(val, idx, P, B, stride_p, stride_b, out_ids,
                                         out_val);
  return hipGetLastError();
}

hipError_t launch_merge_tiles_lse(const float* val, const int32_t* idx, const float* lse,
                                  int32_t S, int32_t B, const float* temperature,
                                  int32_t* out_ids, float* out_val, float* out_lse,
                                  hipStream_t stream) {
  const dim3 grid((B + 3) / 4);
  merge_tiles_lse_kernel<<<grid, 256, 0, stream>>>(val, idx, lse, S, B, temperature, out_ids,
                                                   out_val, out_lse);
  return hipGetLastError();
}

hipError_t launch_merge_group_tiles_lse(const float* val, const int32_t* idx, const float* lse,
                                        int32_t S, int32_t B, const GroupTiles& groups,
                                        const float* temperature, float* out_val,
                                        int32_t* out_idx, float* out_lse, hipStream_t stream) {
  const dim3 grid((B + 3) / 4, groups.n);
  merge_group_tiles_lse_kernel<<<grid, 256, 0, stream>>>(val, idx, lse, S, B, groups, temperature,
                                                         out_val, out_idx, out_lse);
  return hipGetLastError();
}

hipError_t launch_merge_groups_lse(const float* val, const int32_t* idx, const float* lse,
                                   int32_t P, int32_t B, const float* temperature,
                                   uint64_t seed, uint64_t step, int32_t* out_ids,
                                   float* out_val, float* out_lse, hipStream_t stream) {
  const dim3 grid((B + 3) / 4);
  merge_groups_lse_kernel<<<grid, 256, 0, stream>>>(val, idx, lse, P, B, temperature, seed,
                                                    step, out_ids, out_val, out_lse);
  return hipGetLastError();
}

hipError_t launch_debug_noise(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0,
                              int64_t n, uint32_t* bits, float* g, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
  debug_noise_kernel<<<grid, 256, 0, stream>>>(seed, step, row, gv0, n, bits, g);
  return hipGetLastError();
}

hipError_t launch_debug_gumbel(const uint32_t* bits, int64_t n, float* g,
                               hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 65536 ? blocks : 65536));
  debug_gumbel_kernel<<<grid, 256, 0, stream>>>(bits, n, g);
  return hipGetLastError();
}

}  // namespace fs
