// fs_api.hip -- the C ABI of libflashsample (declared in include/flashsample.h).
//
// Every argument is checked here, on the host, before any HIP call; kernels
// assume the checked invariants (D % 8 == 0 and 16-byte aligned operands for
// the 16-byte fragment loads, ids that fit in int32, enough workspace).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/flashsample.h"
#include "fs_internal.hpp"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_forced_config{-1};

fs_status fail(fs_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

fs_status fail(fs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

fs_status hip_fail(hipError_t e, const char* what) {
  return fail(FS_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Testing hook for failure handling: with FS_FAULT_INJECT=launch in the
// environment, every entry point that would launch device work returns
// FS_ERR_HIP once its arguments have passed the checks, before its first
// launch, with the reason in fs_last_error(): the path a failed launch
// takes, without a device and without launching anything.
bool launch_fault_injected() {
  const char* f = getenv("FS_FAULT_INJECT");
  return f != nullptr && std::strcmp(f, "launch") == 0;
}

fs_status injected_failure(const char* who) {
  return fail(FS_ERR_HIP, "%s: launch failure injected (FS_FAULT_INJECT=launch)", who);
}

// Called by every launching entry point once its arguments have passed the
// checks, just before its first HIP call; true when a failure is to be
// injected (and then no HIP call is made).  HIP keeps one pending error per
// host thread: any failed runtime call sets it, and the next hipGetLastError()
// returns and clears it.  The launchers read it right after each launch, so an
// error left pending by an earlier call (the caller's, or one of this
// library's that has already returned its own status) is discarded here
// rather than reported again against this call's launches.
bool start_launches() {
  if (launch_fault_injected()) return true;
  (void)hipGetLastError();
  return false;
}

// Name of a configuration for messages (never a null pointer).
const char* config_label(int cfg) {
  const char* n = fs::fused_config_name(cfg);
  return n != nullptr ? n : "(none)";
}

// Largest batch the batch-tiled kernels can take: their batch blocks (16 or
// more rows each) form the grid's y dimension, at most 65535 blocks.
constexpr int32_t kMaxFusedB = 16 * 65535;
// The unfused baseline's row kernels put one batch row per grid row.
constexpr int32_t kMaxUnfusedB = 65535;

constexpr int64_t kMaxId = 2147483647;  // ids are int32

fs_status check_shape(int32_t B, int32_t D, int32_t V, int32_t vocab_offset) {
  if (B < 0) return fail(FS_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  if (D < 8 || D % 8 != 0)
    return fail(FS_ERR_INVALID_ARG, "D must be a positive multiple of 8 (got %d)", D);
  if (V < 1) return fail(FS_ERR_INVALID_ARG, "V must be >= 1 (got %d)", V);
  if (vocab_offset < 0)
    return fail(FS_ERR_INVALID_ARG, "vocab_offset must be >= 0 (got %d)", vocab_offset);
  if (static_cast<int64_t>(vocab_offset) + V > kMaxId)
    return fail(FS_ERR_INVALID_ARG, "vocab_offset + V exceeds 2^31 - 1 (%d + %d)", vocab_offset,
                V);
  return FS_OK;
}

// workspace == kNoWorkspace: the call uses the library's scratch array.
const void* const kNoWorkspace = reinterpret_cast<const void*>(~uintptr_t{0} & ~uintptr_t{255});

fs_status check_sample_args(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                            int32_t vocab_offset, const float* temperature, const void* out_a,
                            const void* out_b, const void* workspace) {
  fs_status s = check_shape(B, D, V, vocab_offset);
  if (s != FS_OK || B == 0) return s;
  if (!h || !W || !temperature || !out_a || !out_b || !workspace)
    return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(h, 16) || !aligned(W, 16))
    return fail(FS_ERR_INVALID_ARG, "h and W must be 16-byte aligned");
  if (!aligned(temperature, 4) || !aligned(out_a, 4) || !aligned(out_b, 4))
    return fail(FS_ERR_INVALID_ARG, "temperature and outputs must be 4-byte aligned");
  if (!aligned(workspace, 256)) return fail(FS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return FS_OK;
}

// ---- scratch array of the allocation-free entry point ----
// Tile partials of fs_sample_packed_noalloc live here instead of in a caller
// workspace.  Each device the library runs on holds its own copy until the
// process ends; every call on a device shares it, so calls that overlap on
// one device race.  Nothing in it needs to start at zero: a call writes every
// partial it reads.
constexpr size_t kScratchBytes = size_t{8} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (the array's name is a host-side stand-in, not a device address).
fs_status scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FS_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                kMaxDevices);
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FS_OK;
}

// Most vocabulary blocks any configuration launches: blocks of at least
// kMinRowsPerBlock rows over a grid of V rows shifted by vocab_offset mod 4
// (< 4) rows.
size_t max_splits(int32_t V) {
  return (static_cast<size_t>(V) + 3 + fs::kMinRowsPerBlock - 1) / fs::kMinRowsPerBlock;
}

// Workspace: per-tile partial values, ids and log-sum-exps, each [B][S].
size_t fused_workspace(int32_t B, int32_t V) {
  return 3 * fs::round_up(sizeof(float) * B * max_splits(V), 256);
}

// Event pairs around fused-kernel launches (fs_profile_enable / _read).
struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> events;  // start, stop, start, stop, ...
  int used = 0;
};
Profiler g_prof;

void destroy_events() {
  for (hipEvent_t e : g_prof.events) (void)hipEventDestroy(e);
  g_prof.events.clear();
  g_prof.used = 0;
}

int choose_config(int32_t B, int32_t D, int32_t V, bool packed = false) {
  const int forced = g_forced_config.load(std::memory_order_relaxed);
  return forced >= 0 ? forced : fs::fused_auto_config(B, D, V, packed);
}

// Shared body of fs_sample / fs_sample_partial / fs_sample_partial_lse
// (out_lse non-null: also the per-row log-sum-exp of the scaled logits).
fs_status run_fused(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                    int32_t vocab_offset, const float* temperature, uint64_t seed,
                    uint64_t step, int32_t* out_ids, float* out_val, float* out_lse,
                    void* workspace, size_t workspace_bytes, void* stream, const char* who,
                    bool w_packed = false) {
  if (out_lse && !aligned(out_lse, 4))
    return fail(FS_ERR_INVALID_ARG, "%s: partial_lse must be 4-byte aligned", who);
  fs_status s = check_sample_args(h, W, B, D, V, vocab_offset, temperature, out_ids, out_val,
                                  workspace);
  if (s != FS_OK || B == 0) return s;
  const size_t need = fused_workspace(B, V);
  if (workspace != kNoWorkspace && workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu required", who,
                workspace_bytes, need);
  if (w_packed && D % 32 != 0)
    return fail(FS_ERR_INVALID_ARG, "%s: D must be a multiple of 32 (got %d)", who, D);
  if (B > kMaxFusedB)
    return fail(FS_ERR_UNSUPPORTED, "%s: B=%d exceeds the %d batch rows one call can take", who,
                B, kMaxFusedB);
  const int cfg = choose_config(B, D, V, w_packed);
  if (!fs::fused_config_supports(cfg, B, D))
    return fail(FS_ERR_UNSUPPORTED, "%s: forced configuration %s does not support B=%d, D=%d",
                who, config_label(cfg), B, D);
  if (w_packed && !fs::fused_config_reads_packed(cfg))
    return fail(FS_ERR_UNSUPPORTED, "%s: configuration %s for B=%d, D=%d, V=%d has no packed-W kernel",
                who, config_label(cfg), B, D, V);
  // Split capacity of the partial layout: a caller workspace is sized for the
  // most splits any configuration can launch; the scratch array for the
  // chosen configuration's (blocks of its row count over a grid shifted by
  // fewer than 4 rows).
  size_t S = max_splits(V);
  if (workspace == kNoWorkspace) {
    const size_t rows = static_cast<size_t>(fs::fused_rows_per_block(cfg));
    S = (static_cast<size_t>(V) + 3 + rows - 1) / rows;
    const size_t need = (out_lse ? 3 : 2) * fs::round_up(sizeof(float) * B * S, 256);
    if (need > kScratchBytes)
      return fail(FS_ERR_WORKSPACE,
                  "%s: B=%d, V=%d needs %zu bytes of partials, beyond the %zu-byte scratch array",
                  who, B, V, need, kScratchBytes);
    if (start_launches()) return injected_failure(who);
    const fs_status st = scratch_address(&workspace);
    if (st != FS_OK) return st;
  } else if (start_launches()) {
    return injected_failure(who);
  }
  fs::SampleArgs a;
  a.h = static_cast<const __bf16*>(h);
  a.W = static_cast<const __bf16*>(W);
  a.B = B;
  a.D = D;
  a.V = V;
  a.vocab_offset = vocab_offset;
  a.temperature = temperature;
  a.seed = seed;
  a.step = step;
  a.part_val = static_cast<float*>(workspace);
  const size_t region = fs::round_up(sizeof(float) * B * S, 256);
  a.part_idx = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + region);
  a.part_lse = out_lse ? reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * region)
                       : nullptr;
  a.S = 0;
  a.w_packed = w_packed;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (g_prof.on.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    const size_t k = 2 * static_cast<size_t>(g_prof.used);
    const bool rec = k + 1 < g_prof.events.size();
    if (rec && (e = hipEventRecord(g_prof.events[k], st)) != hipSuccess)
      return hip_fail(e, "profile event");
    e = fs::launch_fused(cfg, a, st);
    if (e != hipSuccess) return hip_fail(e, "fused sampler launch");
    if (rec) {
      if ((e = hipEventRecord(g_prof.events[k + 1], st)) != hipSuccess)
        return hip_fail(e, "profile event");
      ++g_prof.used;
    }
  } else {
    e = fs::launch_fused(cfg, a, st);
    if (e != hipSuccess) return hip_fail(e, "fused sampler launch");
  }
  e = out_lse ? fs::launch_merge_tiles_lse(a.part_val, a.part_idx, a.part_lse, a.S, B,
                                           temperature, out_ids, out_val, out_lse, st)
              : fs::launch_merge(a.part_val, a.part_idx, a.S, B, 1, a.S, out_ids, out_val, st);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  if (getenv("FS_LOG"))
    fprintf(stderr, "[flashsample] %s B=%d D=%d V=%d config=%s splits=%d\n", who, B, D, V,
            config_label(cfg), a.S);
  return FS_OK;
}

// ---- grouped sampler in one launch ----
// Most vocabulary blocks a grouped launch over G groups can have: each group's
// blocks (at least 16 rows) start up to 3 rows before its first row.
size_t max_splits_groups(int32_t V, int32_t G) {
  return (static_cast<size_t>(V) + 18 * static_cast<size_t>(G)) / fs::kMinRowsPerBlock + 1;
}

size_t groups_workspace(int32_t B, int32_t V, int32_t G) {
  return 3 * fs::round_up(sizeof(float) * B * max_splits_groups(V, G), 256);
}

// Shared body of fs_sample_groups_lse / fs_sample_groups_lse_packed.
fs_status run_groups(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                     int32_t vocab_offset, const float* temperature, uint64_t seed, uint64_t step,
                     const int32_t* cuts, int32_t G, float* partial_val, int32_t* partial_idx,
                     float* partial_lse, void* workspace, size_t workspace_bytes, void* stream,
                     bool packed, const char* who) {
  fs_status s = check_sample_args(h, W, B, D, V, vocab_offset, temperature, partial_idx,
                                  partial_val, workspace);
  if (s != FS_OK) return s;
  if (!cuts) return fail(FS_ERR_INVALID_ARG, "%s: null cuts", who);
  if (G < 1 || G > fs::kMaxGroups)
    return fail(FS_ERR_INVALID_ARG, "%s: n_groups must be in [1, %d] (got %d)", who, fs::kMaxGroups,
                G);
  if (cuts[0] != 0 || cuts[G] != V)
    return fail(FS_ERR_INVALID_ARG, "%s: cuts must start at 0 and end at V=%d (got %d .. %d)", who,
                V, cuts[0], cuts[G]);
  for (int32_t g = 0; g < G; ++g)
    if (cuts[g + 1] <= cuts[g])
      return fail(FS_ERR_INVALID_ARG, "%s: cuts must increase strictly (cuts[%d]=%d, cuts[%d]=%d)",
                  who, g, cuts[g], g + 1, cuts[g + 1]);
  if (B == 0) return FS_OK;
  if (!partial_lse) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(partial_lse, 4))
    return fail(FS_ERR_INVALID_ARG, "%s: partial_lse must be 4-byte aligned", who);
  if (packed) {
    if (D % 32 != 0)
      return fail(FS_ERR_INVALID_ARG, "%s: D must be a multiple of 32 (got %d)", who, D);
    for (int32_t g = 1; g < G; ++g)
      if (cuts[g] % 16 != 0)
        return fail(FS_ERR_INVALID_ARG, "%s: group starts must be multiples of 16 (cuts[%d]=%d)",
                    who, g, cuts[g]);
  }
  if (B > kMaxFusedB)
    return fail(FS_ERR_UNSUPPORTED, "%s: B=%d exceeds the %d batch rows one call can take", who,
                B, kMaxFusedB);
  const size_t need = groups_workspace(B, V, G);
  if (workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu required", who,
                workspace_bytes, need);
  const int cfg = choose_config(B, D, V, packed);
  if (!fs::fused_config_supports(cfg, B, D))
    return fail(FS_ERR_UNSUPPORTED, "%s: forced configuration %s does not support B=%d, D=%d",
                who, config_label(cfg), B, D);
  if (packed && !fs::fused_config_reads_packed(cfg))
    return fail(FS_ERR_UNSUPPORTED, "%s: configuration %s has no packed-W kernel", who,
                config_label(cfg));
  if (start_launches()) return injected_failure(who);
  const size_t S = max_splits_groups(V, G);
  const size_t region = fs::round_up(sizeof(float) * B * S, 256);
  char* ws = static_cast<char*>(workspace);
  fs::SampleArgs a;
  a.h = static_cast<const __bf16*>(h);
  a.W = static_cast<const __bf16*>(W);
  a.B = B;
  a.D = D;
  a.V = V;
  a.vocab_offset = vocab_offset;
  a.temperature = temperature;
  a.seed = seed;
  a.step = step;
  a.part_val = reinterpret_cast<float*>(ws);
  a.part_idx = reinterpret_cast<int32_t*>(ws + region);
  a.part_lse = reinterpret_cast<float*>(ws + 2 * region);
  a.S = 0;
  a.w_packed = packed;
  a.n_groups = G;
  for (int32_t g = 0; g <= G; ++g) a.grp_rows[g] = cuts[g];
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fs::launch_fused(cfg, a, st);
  if (e != hipSuccess) return hip_fail(e, "fused sampler launch");
  fs::GroupTiles gt;
  gt.n = G;
  for (int32_t g = 0; g <= G; ++g) gt.t[g] = a.grp_tiles[g];
  for (int32_t g = 0; g < G; ++g)
    gt.end[g] = a.grp_span > 0 ? std::min(a.grp_tiles[g + 1], a.grp_tiles[g] + a.grp_span)
                               : a.grp_tiles[g + 1];
  e = fs::launch_merge_group_tiles_lse(a.part_val, a.part_idx, a.part_lse, a.S, B, gt, temperature,
                                       partial_val, partial_idx, partial_lse, st);
  if (e != hipSuccess) return hip_fail(e, "group merge launch");
  if (getenv("FS_LOG"))
    fprintf(stderr, "[flashsample] %s B=%d D=%d V=%d groups=%d config=%s splits=%d\n", who, B, D,
            V, G, config_label(cfg), a.S);
  return FS_OK;
}

// ---- online sampler ----
constexpr int32_t kMaxChunks = 1 << 16;
// Longest rows for which the bound's margin 1 + 2^-8 covers the device's fp32
// logit rounding (about D * 2^-24 relative).
constexpr int32_t kMaxOnlineD = 32768;

fs_status check_cuts(const int32_t* cuts, int32_t n_chunks, int32_t V, const char* who) {
  if (!cuts) return fail(FS_ERR_INVALID_ARG, "%s: null cuts", who);
  if (n_chunks < 1 || n_chunks > kMaxChunks)
    return fail(FS_ERR_INVALID_ARG, "%s: n_chunks must be in [1, %d] (got %d)", who, kMaxChunks,
                n_chunks);
  if (cuts[0] != 0 || cuts[n_chunks] != V)
    return fail(FS_ERR_INVALID_ARG, "%s: cuts must start at 0 and end at V=%d (got %d .. %d)",
                who, V, cuts[0], cuts[n_chunks]);
  for (int32_t c = 0; c < n_chunks; ++c)
    if (cuts[c + 1] <= cuts[c])
      return fail(FS_ERR_INVALID_ARG, "%s: cuts must increase strictly (cuts[%d]=%d, cuts[%d]=%d)",
                  who, c, cuts[c], c + 1, cuts[c + 1]);
  return FS_OK;
}

size_t online_bounds_workspace(int32_t V, int32_t n_chunks) {
  return fs::round_up(sizeof(double) * V, 256) + fs::round_up(sizeof(double) * n_chunks, 256);
}

// fused partials for the longest chunk (at most V rows), then |h_b| (fp64),
// final flags and one live count per chunk
size_t online_workspace(int32_t B, int32_t V, int32_t n_chunks) {
  return fused_workspace(B, V) + fs::round_up(sizeof(double) * B, 256) +
         fs::round_up(sizeof(int32_t) * B, 256) + fs::round_up(sizeof(int32_t) * n_chunks, 256);
}

// Shared body of fs_sample_online / fs_sample_online_packed (W in fragment
// order: every chunk starts on a 16-row group of the packed layout).
static fs_status run_online(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                            int32_t vocab_offset, const float* temperature, uint64_t seed,
                            uint64_t step, const int32_t* cuts, int32_t n_chunks,
                            const double* later_norm, int32_t* out_ids, float* out_maxval,
                            int32_t* out_chunks, void* workspace, size_t workspace_bytes,
                            void* stream, bool packed, const char* who) {
  fs_status s = check_sample_args(h, W, B, D, V, vocab_offset, temperature, out_ids, out_maxval,
                                  workspace);
  if (s != FS_OK) return s;
  if ((s = check_cuts(cuts, n_chunks, V, who)) != FS_OK) return s;
  if (B == 0) return FS_OK;
  if (!out_chunks || !later_norm) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(out_chunks, 4) || !aligned(later_norm, 8))
    return fail(FS_ERR_INVALID_ARG, "out_chunks must be 4-byte and later_norm 8-byte aligned");
  if (packed) {
    if (D % 32 != 0)
      return fail(FS_ERR_INVALID_ARG, "%s: D must be a multiple of 32 (got %d)", who, D);
    for (int32_t c = 1; c < n_chunks; ++c)
      if (cuts[c] % 16 != 0)
        return fail(FS_ERR_INVALID_ARG, "%s: chunk starts must be multiples of 16 (cuts[%d]=%d)",
                    who, c, cuts[c]);
  }
  if (D > kMaxOnlineD)
    return fail(FS_ERR_UNSUPPORTED, "%s: D=%d exceeds %d, where the bound's rounding margin holds",
                who, D, kMaxOnlineD);
  if (B > kMaxFusedB)
    return fail(FS_ERR_UNSUPPORTED, "%s: B=%d exceeds the %d batch rows one call can take", who,
                B, kMaxFusedB);
  const size_t need = online_workspace(B, V, n_chunks);
  if (workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "%s: workspace of %zu bytes is below the %zu required", who,
                workspace_bytes, need);
  // the chunks' configurations, checked before anything is launched
  for (int32_t c = 0; c < n_chunks; ++c) {
    const int cfg = choose_config(B, D, cuts[c + 1] - cuts[c], packed);
    if (!fs::fused_config_supports(cfg, B, D))
      return fail(FS_ERR_UNSUPPORTED, "%s: forced configuration %s does not support B=%d, D=%d",
                  who, config_label(cfg), B, D);
    if (packed && !fs::fused_config_reads_packed(cfg))
      return fail(FS_ERR_UNSUPPORTED, "%s: configuration %s has no packed-W kernel", who,
                  config_label(cfg));
  }
  if (start_launches()) return injected_failure(who);
  const size_t S = max_splits(V);
  const size_t region = fs::round_up(sizeof(float) * B * S, 256);
  char* ws = static_cast<char*>(workspace);
  float* part_val = reinterpret_cast<float*>(ws);
  int32_t* part_idx = reinterpret_cast<int32_t*>(ws + region);
  char* tail = ws + fused_workspace(B, V);
  double* hnorm = reinterpret_cast<double*>(tail);
  tail += fs::round_up(sizeof(double) * B, 256);
  int32_t* done = reinterpret_cast<int32_t*>(tail);
  tail += fs::round_up(sizeof(int32_t) * B, 256);
  int32_t* live = reinterpret_cast<int32_t*>(tail);
  // largest value of the Gumbel map, at the top word: u = 1 - 2^-33
  const double g_max = -std::log(-std::log1p(-0x1p-33));
  const double margin = 1.0 + 0x1p-8;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = fs::launch_online_init(static_cast<const __bf16*>(h), B, D, n_chunks, hnorm,
                                        done, live, out_ids, out_maxval, out_chunks, st);
  if (e != hipSuccess) return hip_fail(e, "online init launch");
  for (int32_t c = 0; c < n_chunks; ++c) {
    fs::SampleArgs a;
    a.h = static_cast<const __bf16*>(h);
    // a packed chunk starts at group cuts[c] / 16 of 16 rows x D
    a.W = static_cast<const __bf16*>(W) + static_cast<size_t>(cuts[c]) * D;
    a.B = B;
    a.D = D;
    a.V = cuts[c + 1] - cuts[c];
    a.vocab_offset = vocab_offset + cuts[c];
    a.temperature = temperature;
    a.seed = seed;
    a.step = step;
    a.part_val = part_val;
    a.part_idx = part_idx;
    a.part_lse = nullptr;
    a.S = 0;
    a.live = c > 0 ? live + (c - 1) : nullptr;
    a.w_packed = packed;
    e = fs::launch_fused(choose_config(B, D, a.V, packed), a, st);
    if (e != hipSuccess) return hip_fail(e, "fused sampler launch");
    e = fs::launch_online_step(part_val, part_idx, a.S, B, c, n_chunks, later_norm, hnorm,
                               temperature, g_max, margin, done, live, out_ids, out_maxval,
                               out_chunks, st);
    if (e != hipSuccess) return hip_fail(e, "online step launch");
  }
  return FS_OK;
}

// Shared body of fs_online_bounds / fs_online_bounds_packed.
static fs_status run_online_bounds(const void* W, int32_t V, int32_t D, int32_t vocab_offset,
                                   const int32_t* cuts, int32_t n_chunks, double* later_norm,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   bool packed) {
  fs_status s = check_shape(1, D, V, vocab_offset);
  if (s != FS_OK) return s;
  if (packed && D % 32 != 0)
    return fail(FS_ERR_INVALID_ARG, "fs_online_bounds_packed: D must be a multiple of 32 (got %d)", D);
  if ((s = check_cuts(cuts, n_chunks, V, "fs_online_bounds")) != FS_OK) return s;
  if (!W || !later_norm || !workspace) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(W, 16)) return fail(FS_ERR_INVALID_ARG, "W must be 16-byte aligned");
  if (!aligned(later_norm, 8)) return fail(FS_ERR_INVALID_ARG, "later_norm must be 8-byte aligned");
  if (!aligned(workspace, 256)) return fail(FS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = online_bounds_workspace(V, n_chunks);
  if (workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "fs_online_bounds: workspace of %zu bytes is below the %zu required",
                workspace_bytes, need);
  if (start_launches()) return injected_failure("fs_online_bounds");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  double* norms = static_cast<double*>(workspace);
  double* chunk_max = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                                fs::round_up(sizeof(double) * V, 256));
  hipError_t e = packed ? fs::launch_packed_row_norms(static_cast<const __bf16*>(W), V, D,
                                                       vocab_offset, norms, st)
                        : fs::launch_row_norms(static_cast<const __bf16*>(W), V, D, norms, st);
  if (e != hipSuccess) return hip_fail(e, "row norm launch");
  for (int32_t c = 0; c < n_chunks; ++c) {
    e = fs::launch_max_reduce(norms + cuts[c], cuts[c + 1] - cuts[c], chunk_max + c, st);
    if (e != hipSuccess) return hip_fail(e, "chunk norm launch");
  }
  e = fs::launch_suffix_max(chunk_max, n_chunks, later_norm, st);
  if (e != hipSuccess) return hip_fail(e, "suffix max launch");
  return FS_OK;
}

}  // namespace

extern "C" {

size_t fs_workspace_bytes(int32_t B, int32_t D, int32_t V) {
  if (check_shape(B, D, V, 0) != FS_OK) return 0;
  return fused_workspace(B, V);
}

size_t fs_unfused_workspace_bytes(int32_t B, int32_t D, int32_t V) {
  if (check_shape(B, D, V, 0) != FS_OK) return 0;
  return fs::unfused_workspace_bytes(B, V);
}

fs_status fs_sample(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                    int32_t vocab_offset, const float* temperature, uint64_t seed,
                    uint64_t step, int32_t* out_ids, float* out_maxval, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return run_fused(h, W, B, D, V, vocab_offset, temperature, seed, step, out_ids, out_maxval,
                   nullptr, workspace, workspace_bytes, stream, "fs_sample");
}

size_t fs_packed_weights_bytes(int32_t V, int32_t D, int32_t vocab_offset) {
  if (check_shape(1, D, V, vocab_offset) != FS_OK || D % 32 != 0) return 0;
  return static_cast<size_t>(fs::packed_groups(V, vocab_offset)) * 16 * D * sizeof(uint16_t);
}

fs_status fs_pack_weights(const void* W, int32_t V, int32_t D, int32_t vocab_offset,
                          void* W_packed, size_t packed_bytes, void* stream) {
  fs_status s = check_shape(1, D, V, vocab_offset);
  if (s != FS_OK) return s;
  if (D % 32 != 0)
    return fail(FS_ERR_INVALID_ARG, "fs_pack_weights: D must be a multiple of 32 (got %d)", D);
  if (!W || !W_packed) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(W, 16) || !aligned(W_packed, 16))
    return fail(FS_ERR_INVALID_ARG, "W and W_packed must be 16-byte aligned");
  const size_t need = fs_packed_weights_bytes(V, D, vocab_offset);
  if (packed_bytes < need)
    return fail(FS_ERR_WORKSPACE, "fs_pack_weights: %zu bytes for W_packed, %zu required",
                packed_bytes, need);
  if (start_launches()) return injected_failure("fs_pack_weights");
  hipError_t e = fs::launch_pack_weights(static_cast<const __bf16*>(W), V, D, vocab_offset,
                                         static_cast<__bf16*>(W_packed),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return FS_OK;
}

fs_status fs_sample_packed(const void* h, const void* W_packed, int32_t B, int32_t D, int32_t V,
                           int32_t vocab_offset, const float* temperature, uint64_t seed,
                           uint64_t step, int32_t* out_ids, float* out_maxval, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_fused(h, W_packed, B, D, V, vocab_offset, temperature, seed, step, out_ids,
                   out_maxval, nullptr, workspace, workspace_bytes, stream, "fs_sample_packed",
                   true);
}

fs_status fs_sample_packed_noalloc(const void* h, const void* W_packed, int32_t B, int32_t D,
                                   int32_t V, int32_t vocab_offset, const float* temperature,
                                   uint64_t seed, uint64_t step, int32_t* out_ids,
                                   float* out_maxval, void* stream) {
  return run_fused(h, W_packed, B, D, V, vocab_offset, temperature, seed, step, out_ids,
                   out_maxval, nullptr, const_cast<void*>(kNoWorkspace), 0, stream,
                   "fs_sample_packed_noalloc", true);
}

fs_status fs_sample_partial(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                            int32_t vocab_offset, const float* temperature, uint64_t seed,
                            uint64_t step, float* partial_val, int32_t* partial_idx,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return run_fused(h, W, B, D, V, vocab_offset, temperature, seed, step, partial_idx,
                   partial_val, nullptr, workspace, workspace_bytes, stream, "fs_sample_partial");
}

fs_status fs_sample_partial_lse(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                                int32_t vocab_offset, const float* temperature, uint64_t seed,
                                uint64_t step, float* partial_val, int32_t* partial_idx,
                                float* partial_lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (B > 0 && !partial_lse) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  return run_fused(h, W, B, D, V, vocab_offset, temperature, seed, step, partial_idx,
                   partial_val, partial_lse, workspace, workspace_bytes, stream,
                   "fs_sample_partial_lse");
}

fs_status fs_sample_partial_lse_packed(const void* h, const void* W_packed, int32_t B, int32_t D,
                                       int32_t V, int32_t vocab_offset, const float* temperature,
                                       uint64_t seed, uint64_t step, float* partial_val,
                                       int32_t* partial_idx, float* partial_lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  if (B > 0 && !partial_lse) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  return run_fused(h, W_packed, B, D, V, vocab_offset, temperature, seed, step, partial_idx,
                   partial_val, partial_lse, workspace, workspace_bytes, stream,
                   "fs_sample_partial_lse_packed", true);
}

size_t fs_groups_workspace_bytes(int32_t B, int32_t D, int32_t V, int32_t n_groups) {
  if (check_shape(B, D, V, 0) != FS_OK || n_groups < 1 || n_groups > fs::kMaxGroups) return 0;
  return groups_workspace(B, V, n_groups);
}

fs_status fs_sample_groups_lse(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                               int32_t vocab_offset, const float* temperature, uint64_t seed,
                               uint64_t step, const int32_t* cuts, int32_t n_groups,
                               float* partial_val, int32_t* partial_idx, float* partial_lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return run_groups(h, W, B, D, V, vocab_offset, temperature, seed, step, cuts, n_groups,
                    partial_val, partial_idx, partial_lse, workspace, workspace_bytes, stream,
                    false, "fs_sample_groups_lse");
}

fs_status fs_sample_groups_lse_packed(const void* h, const void* W_packed, int32_t B, int32_t D,
                                      int32_t V, int32_t vocab_offset, const float* temperature,
                                      uint64_t seed, uint64_t step, const int32_t* cuts,
                                      int32_t n_groups, float* partial_val, int32_t* partial_idx,
                                      float* partial_lse, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return run_groups(h, W_packed, B, D, V, vocab_offset, temperature, seed, step, cuts, n_groups,
                    partial_val, partial_idx, partial_lse, workspace, workspace_bytes, stream, true,
                    "fs_sample_groups_lse_packed");
}

fs_status fs_merge_lse(const float* partial_val, const int32_t* partial_idx,
                       const float* partial_lse, int32_t P, int32_t B,
                       const float* temperature, uint64_t seed, uint64_t step,
                       int32_t* out_ids, float* out_maxval, float* out_lse, void* stream) {
  if (P < 1) return fail(FS_ERR_INVALID_ARG, "P must be >= 1 (got %d)", P);
  if (B < 0) return fail(FS_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  if (B == 0) return FS_OK;
  if (!partial_val || !partial_idx || !partial_lse || !temperature || !out_ids || !out_maxval ||
      !out_lse)
    return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(partial_val, 4) || !aligned(partial_idx, 4) || !aligned(partial_lse, 4) ||
      !aligned(temperature, 4) || !aligned(out_ids, 4) || !aligned(out_maxval, 4) ||
      !aligned(out_lse, 4))
    return fail(FS_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  if (static_cast<int64_t>(P) * B > (int64_t{1} << 40))
    return fail(FS_ERR_INVALID_ARG, "P * B too large");
  if (start_launches()) return injected_failure("fs_merge_lse");
  hipError_t e = fs::launch_merge_groups_lse(partial_val, partial_idx, partial_lse, P, B,
                                             temperature, seed, step, out_ids, out_maxval,
                                             out_lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "grouped merge launch");
  return FS_OK;
}

size_t fs_online_bounds_workspace_bytes(int32_t V, int32_t n_chunks) {
  if (V < 1 || n_chunks < 1 || n_chunks > kMaxChunks) return 0;
  return online_bounds_workspace(V, n_chunks);
}

size_t fs_online_workspace_bytes(int32_t B, int32_t D, int32_t V, int32_t n_chunks) {
  if (check_shape(B, D, V, 0) != FS_OK || n_chunks < 1 || n_chunks > kMaxChunks) return 0;
  return online_workspace(B, V, n_chunks);
}

fs_status fs_online_bounds(const void* W, int32_t V, int32_t D, const int32_t* cuts,
                           int32_t n_chunks, double* later_norm, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run_online_bounds(W, V, D, 0, cuts, n_chunks, later_norm, workspace, workspace_bytes,
                           stream, false);
}

fs_status fs_online_bounds_packed(const void* W_packed, int32_t V, int32_t D,
                                  int32_t vocab_offset, const int32_t* cuts, int32_t n_chunks,
                                  double* later_norm, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return run_online_bounds(W_packed, V, D, vocab_offset, cuts, n_chunks, later_norm, workspace,
                           workspace_bytes, stream, true);
}

fs_status fs_sample_online(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                           int32_t vocab_offset, const float* temperature, uint64_t seed,
                           uint64_t step, const int32_t* cuts, int32_t n_chunks,
                           const double* later_norm, int32_t* out_ids, float* out_maxval,
                           int32_t* out_chunks, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return run_online(h, W, B, D, V, vocab_offset, temperature, seed, step, cuts, n_chunks,
                    later_norm, out_ids, out_maxval, out_chunks, workspace, workspace_bytes,
                    stream, false, "fs_sample_online");
}

fs_status fs_sample_online_packed(const void* h, const void* W_packed, int32_t B, int32_t D,
                                  int32_t V, int32_t vocab_offset, const float* temperature,
                                  uint64_t seed, uint64_t step, const int32_t* cuts,
                                  int32_t n_chunks, const double* later_norm, int32_t* out_ids,
                                  float* out_maxval, int32_t* out_chunks, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return run_online(h, W_packed, B, D, V, vocab_offset, temperature, seed, step, cuts, n_chunks,
                    later_norm, out_ids, out_maxval, out_chunks, workspace, workspace_bytes,
                    stream, true, "fs_sample_online_packed");
}

fs_status fs_merge(const float* partial_val, const int32_t* partial_idx, int32_t P, int32_t B,
                   int32_t* out_ids, float* out_maxval, void* stream) {
  if (P < 1) return fail(FS_ERR_INVALID_ARG, "P must be >= 1 (got %d)", P);
  if (B < 0) return fail(FS_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  if (B == 0) return FS_OK;
  if (!partial_val || !partial_idx || !out_ids || !out_maxval)
    return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(partial_val, 4) || !aligned(partial_idx, 4) || !aligned(out_ids, 4) ||
      !aligned(out_maxval, 4))
    return fail(FS_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  if (static_cast<int64_t>(P) * B > (int64_t{1} << 40))
    return fail(FS_ERR_INVALID_ARG, "P * B too large");
  if (start_launches()) return injected_failure("fs_merge");
  hipError_t e = fs::launch_merge(partial_val, partial_idx, P, B, B, 1, out_ids, out_maxval,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return FS_OK;
}

fs_status fs_sample_unfused(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                            int32_t vocab_offset, const float* temperature, uint64_t seed,
                            uint64_t step, int32_t* out_ids, float* out_maxval,
                            void* workspace, size_t workspace_bytes, void* stream) {
  fs_status s = check_sample_args(h, W, B, D, V, vocab_offset, temperature, out_ids,
                                  out_maxval, workspace);
  if (s != FS_OK || B == 0) return s;
  if (B > kMaxUnfusedB)
    return fail(FS_ERR_UNSUPPORTED, "fs_sample_unfused: B=%d exceeds the %d batch rows one call can take",
                B, kMaxUnfusedB);
  const size_t need = fs::unfused_workspace_bytes(B, V);
  if (workspace_bytes < need)
    return fail(FS_ERR_WORKSPACE, "fs_sample_unfused: workspace of %zu bytes is below the %zu required",
                workspace_bytes, need);
  if (start_launches()) return injected_failure("fs_sample_unfused");
  fs::SampleArgs a;
  a.h = static_cast<const __bf16*>(h);
  a.W = static_cast<const __bf16*>(W);
  a.B = B;
  a.D = D;
  a.V = V;
  a.vocab_offset = vocab_offset;
  a.temperature = temperature;
  a.seed = seed;
  a.step = step;
  a.part_val = nullptr;
  a.part_lse = nullptr;
  a.part_idx = nullptr;
  a.S = 0;
  hipError_t e = fs::launch_unfused(a, out_ids, out_maxval, workspace,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "unfused sampler launch");
  return FS_OK;
}

fs_status fs_debug_noise(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0, int64_t n,
                         uint32_t* out_bits, float* out_gumbel, void* stream) {
  if (n < 0) return fail(FS_ERR_INVALID_ARG, "n must be >= 0");
  if (static_cast<uint64_t>(gv0) + static_cast<uint64_t>(n) > (uint64_t{1} << 32))
    return fail(FS_ERR_INVALID_ARG, "gv0 + n exceeds 2^32");
  if (n == 0 || (!out_bits && !out_gumbel)) return FS_OK;
  if ((out_bits && !aligned(out_bits, 4)) || (out_gumbel && !aligned(out_gumbel, 4)))
    return fail(FS_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
  if (start_launches()) return injected_failure("fs_debug_noise");
  hipError_t e = fs::launch_debug_noise(seed, step, row, gv0, n, out_bits, out_gumbel,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "noise launch");
  return FS_OK;
}

fs_status fs_debug_gumbel(const uint32_t* bits, int64_t n, float* out_gumbel, void* stream) {
  if (n < 0) return fail(FS_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return FS_OK;
  if (!bits || !out_gumbel) return fail(FS_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(bits, 4) || !aligned(out_gumbel, 4))
    return fail(FS_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  if (start_launches()) return injected_failure("fs_debug_gumbel");
  hipError_t e = fs::launch_debug_gumbel(bits, n, out_gumbel, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gumbel launch");
  return FS_OK;
}

fs_status fs_profile_enable(int32_t capacity) {
  if (capacity < 0) return fail(FS_ERR_INVALID_ARG, "capacity must be >= 0");
  std::lock_guard<std::mutex> lock(g_prof.mu);
  g_prof.on.store(false, std::memory_order_release);
  destroy_events();
  if (capacity == 0) return FS_OK;
  g_prof.events.resize(2 * static_cast<size_t>(capacity));
  for (auto& ev : g_prof.events) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      ev = nullptr;
      destroy_events();
      return hip_fail(e, "hipEventCreate");
    }
  }
  g_prof.on.store(true, std::memory_order_release);
  return FS_OK;
}

fs_status fs_profile_read(int32_t* launches, double* total_ms, double* min_ms,
                          double* max_ms) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  double tot = 0.0, lo = 0.0, hi = 0.0;
  for (int i = 0; i < g_prof.used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.events[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_prof.events[2 * i], g_prof.events[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    tot += ms;
    lo = (i == 0 || ms < lo) ? ms : lo;
    hi = (i == 0 || ms > hi) ? ms : hi;
  }
  if (launches) *launches = g_prof.used;
  if (total_ms) *total_ms = tot;
  if (min_ms) *min_ms = lo;
  if (max_ms) *max_ms = hi;
  g_prof.used = 0;
  return FS_OK;
}

fs_status fs_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz) {
  if (device < 0) return fail(FS_ERR_INVALID_ARG, "device must be >= 0 (got %d)", device);
  int v = 0;
  hipError_t e;
  if (compute_units) {
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device)) != hipSuccess)
      return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    *compute_units = v;
  }
  if (clock_khz) {
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, device)) != hipSuccess)
      return hip_fail(e, "hipDeviceGetAttribute(ClockRate)");
    *clock_khz = v;
  }
  return FS_OK;
}

int32_t fs_num_configs(void) { return fs::num_fused_configs(); }

const char* fs_config_name(int32_t id) { return fs::fused_config_name(id); }

fs_status fs_force_config(int32_t id) {
  if (id < -1 || id >= fs::num_fused_configs())
    return fail(FS_ERR_INVALID_ARG, "config id %d out of range [-1, %d)", id,
                fs::num_fused_configs());
  g_forced_config.store(id, std::memory_order_relaxed);
  return FS_OK;
}

int32_t fs_selected_config(int32_t B, int32_t D, int32_t V) {
  if (check_shape(B, D, V, 0) != FS_OK) return -1;
  return choose_config(B, D, V);
}

int32_t fs_selected_config_packed(int32_t B, int32_t D, int32_t V) {
  if (check_shape(B, D, V, 0) != FS_OK) return -1;
  return choose_config(B, D, V, true);
}

int32_t fs_selected_config_groups(int32_t B, int32_t D, int32_t V, int32_t packed) {
  if (check_shape(B, D, V, 0) != FS_OK) return -1;
  return choose_config(B, D, V, packed != 0);
}

const char* fs_status_string(fs_status s) {
  // A caller may pass any int: read the code's bits instead of loading an
  // enum value outside its range (undefined behaviour in C++).
  static_assert(sizeof(fs_status) == sizeof(int), "status is int-sized");
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case FS_OK: return "FS_OK";
    case FS_ERR_INVALID_ARG: return "FS_ERR_INVALID_ARG";
    case FS_ERR_UNSUPPORTED: return "FS_ERR_UNSUPPORTED";
    case FS_ERR_WORKSPACE: return "FS_ERR_WORKSPACE";
    case FS_ERR_HIP: return "FS_ERR_HIP";
  }
  return "FS_ERR_UNKNOWN";
}

const char* fs_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
