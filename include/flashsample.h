/*
 * flashsample.h -- C ABI of libflashsample: exact categorical sampling fused
 * into the LM-head matmul, for AMD Instinct MI355X (gfx950).
 *
 * The operation ("FlashSampling: Fast and Memory-Efficient Exact Sampling";
 * wiki summary page, sections "Key claims" and "Method"; arXiv abstract):
 * for each batch row b the library draws one token id from
 * softmax(z_b / T_b), z_b = W h_b, by the Gumbel-Max trick -- the argmax over
 * v of  s[b][v] = z[b][v] / T_b + g[b][v]  with g standard Gumbel noise.  The
 * logits are formed tile by tile on chip, scaled, perturbed and reduced to
 * one (max, argmax) pair per row and per vocabulary tile; a small reduction
 * over tiles returns the id.  The B x V logits never reach device memory.
 *
 * Noise field.  The pages leave the generator open; here it is
 * Philox-4x32-10 (Salmon et al., SC'11).  For batch row b and GLOBAL
 * vocabulary id gv = vocab_offset + v:
 *   x = word (gv mod 4) of Philox4x32_10(counter = {gv / 4, b, step_lo,
 *       step_hi}, key = {seed_lo, seed_hi})
 *   u = (x + 1/2) * 2^-32                   (all 32 bits; 0 < u < 1)
 *   g = -log(-log u)
 * Equal logits therefore tie for the largest score only when two ids draw
 * the same word (about V * 2^-33 of draws).
 * Keying on the global id makes the field independent of tiling and of
 * vocabulary sharding, so per-shard results merge to the unsharded result
 * (wiki summary, "Method", tensor-parallel paragraph).
 *
 * Scores.  s = z * fp32(1/T_b) + g, with z accumulated in fp32 from bf16
 * products.  A row whose temperature is not a positive number (0, -0,
 * negative, NaN) is greedy: s = z (no scaling, no noise).  Ties go to the
 * smaller global id.
 *
 * Conventions for every entry point:
 *   - h is bf16 [B][D] row-major, W is bf16 [V][D] row-major (the layout of
 *     an nn.Linear weight); both device pointers, 16-byte aligned; D % 8 == 0.
 *   - temperature, out_ids, out_maxval, partials: device pointers, 4-byte
 *     aligned.  workspace: device pointer, 256-byte aligned.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous and ordered on that stream; the caller keeps every buffer
 *     alive until the stream has reached the work.
 *   - Ownership: the caller owns all memory.  The library allocates nothing
 *     on the sampling path (the one device array it holds, for
 *     fs_sample_packed_noalloc, is static) and keeps no pointer after
 *     returning; between calls it holds only a forced-configuration switch
 *     (fs_force_config), per-device caches of device facts and launch sizes,
 *     and the profiling recorder (fs_profile_enable).
 *   - Errors: the return code is the only channel.  Arguments are checked on
 *     the host before any HIP call; a rejected call launches nothing and
 *     writes nothing.  FS_ERR_HIP carries the runtime's message in
 *     fs_last_error() (thread-local).  An error that an earlier failed HIP
 *     call left pending in the calling thread is discarded before a call's
 *     first launch, so it is not reported again.  Device-resident values are
 *     not inspected: NaN or infinite entries in h or W give undefined ids.
 *   - B == 0 is a no-op that returns FS_OK (pointers may then be NULL).
 *     The samplers take at most 1048560 (16 * 65535) batch rows per call and
 *     the unfused baseline at most 65535 (the launch grids' row limit);
 *     larger B is FS_ERR_UNSUPPORTED.
 *   - Reentrant: concurrent calls are safe if they use distinct workspaces.
 *   - Failure testing: with FS_FAULT_INJECT=launch in the environment, every
 *     entry point that would launch device work returns FS_ERR_HIP once its
 *     arguments have passed the checks, and launches nothing;
 *     fs_last_error() then names the injection.
 */
#ifndef FLASHSAMPLE_H
#define FLASHSAMPLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FS_API __attribute__((visibility("default")))

typedef enum {
  FS_OK = 0,
  FS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or range */
  FS_ERR_UNSUPPORTED = 2, /* valid request this build cannot run */
  FS_ERR_WORKSPACE = 3,   /* workspace_bytes below the required size */
  FS_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} fs_status;

/* Bytes of workspace fs_sample / fs_sample_partial need for (B, D, V).
 * Returns 0 when the sizes are invalid (see fs_sample). */
FS_API size_t fs_workspace_bytes(int32_t B, int32_t D, int32_t V);

/* Bytes of workspace fs_sample_unfused needs: the materialised fp32 logits
 * and probabilities (2 * B * V * 4 bytes) plus per-row statistics. */
FS_API size_t fs_unfused_workspace_bytes(int32_t B, int32_t D, int32_t V);

/* Sample one token id per batch row (wiki summary, "Method": per-tile
 * maximisers over vocabulary tiles, then the partition argmax).
 *   h            bf16 [B][D]
 *   W            bf16 [V][D]; row v has global id vocab_offset + v
 *   B, D, V      B >= 0; D >= 8, D % 8 == 0; V >= 1
 *   vocab_offset >= 0 and vocab_offset + V <= 2^31 - 1
 *   temperature  fp32 [B]; !(T > 0) selects greedy for that row
 *   seed, step   64-bit noise key and step counter (fresh per decode step)
 *   out_ids      int32 [B]: sampled GLOBAL id per row
 *   out_maxval   fp32 [B]: the winning perturbed score s
 *   workspace    >= fs_workspace_bytes(B, D, V) bytes; contents on entry
 *                are ignored (scratch for per-tile partials)             */
FS_API fs_status fs_sample(const void* h, const void* W, int32_t B, int32_t D, int32_t V,
                    int32_t vocab_offset, const float* temperature, uint64_t seed,
                    uint64_t step, int32_t* out_ids, float* out_maxval,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Fragment-order weights.  The sampler reads W one MFMA operand fragment at
 * a time (16 vocabulary rows x 32 k, 16 bytes per lane); from row-major W
 * each such read takes 64 bytes from each of 16 rows 8 KB apart, which costs
 * HBM page locality.  fs_pack_weights copies W once (at model load) into the
 * fragment order the kernels consume: the vocabulary rows in groups of 16
 * starting at row -(vocab_offset mod 4), each group stored k-step by k-step
 * as 64 pieces of 16 bytes (element ((g * D/32 + s) * 64 + l) * 8 + j holds
 * W[16 g + (l mod 16) - (vocab_offset mod 4)][32 s + 8 (l / 16) + j], zero
 * outside [0, V)).
 *   W            bf16 [V][D], device, 16-byte aligned; D % 32 == 0
 *   vocab_offset the offset the packed weights will be sampled at (only its
 *                value mod 4 shapes the layout)
 *   W_packed     device, 16-byte aligned, >= fs_packed_weights_bytes(V, D,
 *                vocab_offset) bytes (0 for invalid arguments); caller-owned
 * fs_sample_packed takes fs_sample's arguments with W_packed in place of W
 * (packed for the same V, D and vocab_offset mod 4).  Its kernels read the
 * same operand fragments as fs_sample's: run in one configuration
 * (fs_force_config) the two return the same ids and scores bit for bit; the
 * automatic choices may differ (fs_selected_config_packed), and then so may
 * the scores' last bits, within the parity bound of fs_sample.  It runs the
 * persistent, DMA-staged and LDS-staged kernels; a shape whose configuration
 * has no fragment-order kernel (the K-split and streaming loops chosen for
 * small batches at unusual D) returns FS_ERR_UNSUPPORTED.  D % 32 != 0 is
 * FS_ERR_INVALID_ARG. */
FS_API size_t fs_packed_weights_bytes(int32_t V, int32_t D, int32_t vocab_offset);
FS_API fs_status fs_pack_weights(const void* W, int32_t V, int32_t D, int32_t vocab_offset,
                                 void* W_packed, size_t packed_bytes, void* stream);
FS_API fs_status fs_sample_packed(const void* h, const void* W_packed, int32_t B, int32_t D,
                                  int32_t V, int32_t vocab_offset, const float* temperature,
                                  uint64_t seed, uint64_t step, int32_t* out_ids,
                                  float* out_maxval, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* fs_sample_packed without a workspace argument, for callers that cannot
 * allocate device memory around the call (code being captured into a graph,
 * tight serving loops, harnesses that forbid allocation).  The tile partials
 * go to an 8 MiB array the library holds in each device's memory until the
 * process ends; the call allocates nothing.  Its kernels and results are
 * fs_sample_packed's.  Every call on one device shares that array, so calls
 * that overlap on one device (concurrent streams, or several host threads)
 * race and must be serialised by the caller.  A shape whose partials exceed
 * the array (2 * 4 * B * ceil((V + 3) / rows) bytes, rows the chosen
 * configuration's vocabulary rows per block: 16 for the small-batch
 * kernels, 256 or more for the batch-tiled ones) returns FS_ERR_WORKSPACE
 * and launches nothing; other errors as fs_sample_packed. */
FS_API fs_status fs_sample_packed_noalloc(const void* h, const void* W_packed, int32_t B,
                                          int32_t D, int32_t V, int32_t vocab_offset,
                                          const float* temperature, uint64_t seed, uint64_t step,
                                          int32_t* out_ids, float* out_maxval, void* stream);

/* One vocabulary shard's contribution for the grouped / tensor-parallel flow
 * (wiki summary, "Method": each rank reduces its own shard to a per-row
 * (local max, local argmax) pair, and only those pairs are exchanged).
 * Same inputs and semantics as fs_sample over rows [vocab_offset,
 * vocab_offset + V) of the global vocabulary; writes partial_val[b] and
 * partial_idx[b] (GLOBAL ids), i.e. slot p of a P x B partial buffer when
 * the caller passes base + p * B. */
FS_API fs_status fs_sample_partial(const void* h, const void* W, int32_t B, int32_t D,
                            int32_t V, int32_t vocab_offset, const float* temperature,
                            uint64_t seed, uint64_t step, float* partial_val,
                            int32_t* partial_idx, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Cross-part argmax (wiki summary, "Method": the final cross-rank argmax).
 *   partial_val  fp32 [P][B], partial_idx int32 [P][B] (part-major)
 *   P >= 1, B >= 0
 * Per row: the largest value wins; on equal values the smaller id wins.
 * Bit-exact: the result depends only on the set of pairs, not their order. */
FS_API fs_status fs_merge(const float* partial_val, const int32_t* partial_idx, int32_t P,
                   int32_t B, int32_t* out_ids, float* out_maxval, void* stream);

/* Grouped (hierarchical) sampler, one vocabulary group per call (arXiv
 * abstract page and wiki summary, "Key claims": grouped variants for online
 * and tensor-parallel settings are exact by hierarchical factorisation of
 * the categorical distribution; wiki summary, "Method", last paragraph: the
 * online, chunked setting).  As fs_sample_partial, plus
 *   partial_lse  fp32 [B], device: per row the log-sum-exp of the group's
 *                scaled logits, log sum_v exp(z_v * (1/T)); for greedy rows
 *                (T not > 0) the group's largest logit.
 * partial_val / partial_idx are bit-identical to fs_sample_partial's on the
 * same inputs.  Same workspace (fs_workspace_bytes) and errors. */
FS_API fs_status fs_sample_partial_lse(const void* h, const void* W, int32_t B, int32_t D,
                                int32_t V, int32_t vocab_offset, const float* temperature,
                                uint64_t seed, uint64_t step, float* partial_val,
                                int32_t* partial_idx, float* partial_lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/* The same on fragment-order weights (fs_pack_weights, for this group's rows
 * at this vocab_offset mod 4): W_packed in place of W, D % 32 == 0. */
FS_API fs_status fs_sample_partial_lse_packed(const void* h, const void* W_packed, int32_t B,
                                              int32_t D, int32_t V, int32_t vocab_offset,
                                              const float* temperature, uint64_t seed,
                                              uint64_t step, float* partial_val,
                                              int32_t* partial_idx, float* partial_lse,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

/* The grouped sampler's per-group partials for G groups in one launch.  The
 * vocabulary W[0 .. V) is split at the HOST array cuts (0 = cuts[0] <
 * cuts[1] < ... < cuts[G] = V, 1 <= G <= 64); slot g of the outputs (element
 * g * B + b of partial_val / partial_idx / partial_lse, [G][B] part-major as
 * fs_merge_lse reads them) holds what fs_sample_partial_lse would return over
 * W rows [cuts[g], cuts[g+1]) at vocab_offset + cuts[g]: the group's
 * Gumbel-max (value, global id) and its log-sum-exp.  One fused launch covers
 * every group (each group's vocabulary rows are tiled from its own first row,
 * so no tile mixes two groups) and one merge launch fills the slots, instead
 * of G launches each over a slice too short to fill the device.  In one
 * configuration (fs_force_config) the slots' values and ids equal the
 * separate calls bit for bit, and so do the log-sum-exps on the batch-tiled
 * configurations; the persistent ones (small batches) add a group's
 * log-sum-exp partials in another order, equal within rounding.
 *   workspace   >= fs_groups_workspace_bytes(B, D, V, G) bytes (0 for invalid
 *               arguments); contents on entry ignored
 * Errors as fs_sample_partial_lse; a cuts array that does not partition
 * [0, V) or G outside [1, 64] is FS_ERR_INVALID_ARG.  The _packed form reads
 * fragment-order W (fs_pack_weights at the same vocab_offset mod 4) and needs
 * every group start cuts[g] (0 < g < G) to be a multiple of 16. */
FS_API size_t fs_groups_workspace_bytes(int32_t B, int32_t D, int32_t V, int32_t n_groups);
FS_API fs_status fs_sample_groups_lse(const void* h, const void* W, int32_t B, int32_t D,
                                      int32_t V, int32_t vocab_offset, const float* temperature,
                                      uint64_t seed, uint64_t step, const int32_t* cuts,
                                      int32_t n_groups, float* partial_val, int32_t* partial_idx,
                                      float* partial_lse, void* workspace,
                                      size_t workspace_bytes, void* stream);
FS_API fs_status fs_sample_groups_lse_packed(const void* h, const void* W_packed, int32_t B,
                                             int32_t D, int32_t V, int32_t vocab_offset,
                                             const float* temperature, uint64_t seed,
                                             uint64_t step, const int32_t* cuts, int32_t n_groups,
                                             float* partial_val, int32_t* partial_idx,
                                             float* partial_lse, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* Grouped merge: the categorical distribution factorises as
 * P(i) = P(G) P(i | G) with P(G) proportional to exp(LSE_G), and each
 * group's partial already holds a sample of P(i | G).
 *   partial_val, partial_idx, partial_lse  [P][B] (part-major), from
 *                fs_sample_partial_lse, group p in slot p
 *   temperature  fp32 [B], device (greedy rows as in fs_sample)
 *   seed, step   key of the group draws: gamma_p is the Gumbel value of
 *                Philox-4x32-10 word 0 at counter (2^31 | p, row, step low,
 *                step high) under key (seed low, seed high), a counter the
 *                token noise never uses
 * Per row b the group p* = argmax_p (lse_p + gamma_p) (greedy rows:
 * argmax_p lse_p), ties to the smaller p; out_ids[b] / out_maxval[b] are
 * that group's partial, out_lse[b] the row's total log-sum-exp over the
 * groups (greedy rows: the largest lse_p).  All pointers device, 4-byte
 * aligned; P >= 1, B >= 0. */
FS_API fs_status fs_merge_lse(const float* partial_val, const int32_t* partial_idx,
                       const float* partial_lse, int32_t P, int32_t B,
                       const float* temperature, uint64_t seed, uint64_t step,
                       int32_t* out_ids, float* out_maxval, float* out_lse, void* stream);

/* Online (chunked) sampler with early finalisation (wiki summary, "Method",
 * last paragraph: in the online setting the sampler streams over pieces of
 * the vocabulary and may finalise before it has seen them all).  The
 * vocabulary is processed in the chunks W[cuts[c] .. cuts[c+1]), c = 0 ..
 * n_chunks - 1, in order; the running (max, argmax) over the chunks seen so
 * far is the Gumbel-max over them.  The pages state no stopping rule; the one
 * used here follows from Cauchy-Schwarz: row b is final after chunk c once
 * its running best exceeds
 *     (|h_b| * later_norm[c] * fp32(1/T_b) + g_max) * (1 + 2^-8)
 * (greedy rows: |h_b| * later_norm[c] * (1 + 2^-8)), where later_norm[c] is
 * the largest row norm of W over the chunks after c and g_max =
 * -log(-log(1 - 2^-33)) the largest Gumbel value of the noise field.  No later
 * score can overtake such a row, so the ids and scores are those of
 * fs_sample over the whole of W; only the work changes.  Once every row is
 * final the remaining chunks' kernels return without reading their W rows.
 *
 * fs_online_bounds computes later_norm once per weight matrix and chunking:
 *   W            bf16 [V][D], device, 16-byte aligned, D % 8 == 0
 *   cuts         HOST int32 [n_chunks + 1]: 0 = cuts[0] < cuts[1] < ... <
 *                cuts[n_chunks] = V; 1 <= n_chunks <= 65536
 *   later_norm   fp64 [n_chunks], device, 8-byte aligned: later_norm[c] =
 *                max over rows v >= cuts[c+1] of |W_v| (fp64 sums), and
 *                later_norm[n_chunks - 1] = 0
 *   workspace    >= fs_online_bounds_workspace_bytes(V, n_chunks) bytes
 *
 * fs_sample_online takes fs_sample's arguments plus
 *   cuts, n_chunks  as above (HOST array), relative to W row 0: chunk c holds
 *                global ids vocab_offset + cuts[c] .. vocab_offset + cuts[c+1] - 1
 *   later_norm   from fs_online_bounds for the same W and cuts (device)
 *   out_chunks   int32 [B], device: chunks folded into row b's result (the
 *                chunk after which it became final, else n_chunks)
 *   workspace    >= fs_online_workspace_bytes(B, D, V, n_chunks) bytes
 * out_ids / out_maxval as fs_sample.  D <= 32768 (FS_ERR_UNSUPPORTED beyond:
 * the margin 1 + 2^-8 covers the device's fp32 rounding of logits up to that
 * length).  Other errors as fs_sample; a cuts array that does not partition
 * [0, V) is FS_ERR_INVALID_ARG.  Both workspace-size functions return 0 for
 * invalid arguments. */
FS_API size_t fs_online_bounds_workspace_bytes(int32_t V, int32_t n_chunks);
FS_API size_t fs_online_workspace_bytes(int32_t B, int32_t D, int32_t V, int32_t n_chunks);
FS_API fs_status fs_online_bounds(const void* W, int32_t V, int32_t D, const int32_t* cuts,
                                  int32_t n_chunks, double* later_norm, void* workspace,
                                  size_t workspace_bytes, void* stream);
FS_API fs_status fs_sample_online(const void* h, const void* W, int32_t B, int32_t D,
                                  int32_t V, int32_t vocab_offset, const float* temperature,
                                  uint64_t seed, uint64_t step, const int32_t* cuts,
                                  int32_t n_chunks, const double* later_norm, int32_t* out_ids,
                                  float* out_maxval, int32_t* out_chunks, void* workspace,
                                  size_t workspace_bytes, void* stream);
/* The same on fragment-order weights (fs_pack_weights at the same
 * vocab_offset mod 4): W_packed in place of W, every chunk start cuts[c]
 * (0 < c < n_chunks) a multiple of 16, D % 32 == 0 (FS_ERR_INVALID_ARG
 * otherwise).  later_norm comes from fs_online_bounds on the row-major W or
 * from fs_online_bounds_packed on W_packed (same values up to fp64 summation
 * order).  Results as fs_sample_packed over the whole W. */
FS_API fs_status fs_online_bounds_packed(const void* W_packed, int32_t V, int32_t D,
                                         int32_t vocab_offset, const int32_t* cuts,
                                         int32_t n_chunks, double* later_norm, void* workspace,
                                         size_t workspace_bytes, void* stream);
FS_API fs_status fs_sample_online_packed(const void* h, const void* W_packed, int32_t B,
                                         int32_t D, int32_t V, int32_t vocab_offset,
                                         const float* temperature, uint64_t seed, uint64_t step,
                                         const int32_t* cuts, int32_t n_chunks,
                                         const double* later_norm, int32_t* out_ids,
                                         float* out_maxval, int32_t* out_chunks,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* The standard unfused decode step the method replaces (wiki summary,
 * "Method", first paragraph): (1) matmul writing fp32 logits [B][V] to
 * device memory, (2) softmax of z / T writing probabilities, (3)+(4)
 * Gumbel perturbation of log-probabilities and argmax.  Same arguments,
 * noise field and outputs as fs_sample (out_maxval is reported on the
 * s = z / T + g scale by adding back each row's log-normaliser); workspace
 * >= fs_unfused_workspace_bytes(B, D, V).  A baseline for measurement. */
FS_API fs_status fs_sample_unfused(const void* h, const void* W, int32_t B, int32_t D,
                            int32_t V, int32_t vocab_offset, const float* temperature,
                            uint64_t seed, uint64_t step, int32_t* out_ids,
                            float* out_maxval, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Diagnostics: the device noise field, from the same device functions the
 * samplers use.  Writes, for gv = gv0 .. gv0 + n - 1 of one (seed, step,
 * row), the raw Philox word (out_bits, may be NULL) and the Gumbel value g
 * (out_gumbel, may be NULL).  n >= 0; gv0 + n <= 2^32. */
FS_API fs_status fs_debug_noise(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0,
                         int64_t n, uint32_t* out_bits, float* out_gumbel,
                         void* stream);

/* Diagnostics: g = -log(-log u(x)) for n given words (device arrays). */
FS_API fs_status fs_debug_gumbel(const uint32_t* bits, int64_t n, float* out_gumbel,
                          void* stream);

/* Diagnostics: the compute-unit count and the peak shader clock (kHz) the
 * HIP runtime reports for `device`, from which a caller derives the dense
 * MFMA peak it measures against.  Either output may be NULL. */
FS_API fs_status fs_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz);

/* Kernel configurations of the fused sampler.  fs_force_config(id) pins
 * every later fs_sample call in the process to configuration id (0 ..
 * fs_num_configs() - 1); id = -1 restores the automatic choice.  Results do
 * not depend on the configuration.  Not synchronised with concurrent calls. */
FS_API int32_t fs_num_configs(void);
FS_API const char* fs_config_name(int32_t id);
FS_API fs_status fs_force_config(int32_t id);
/* Configuration fs_sample would use for batch size B (after forcing), the
 * one fs_sample_packed would use, and the one fs_sample_groups_lse (packed
 * != 0: fs_sample_groups_lse_packed) would use over a V-row vocabulary (the
 * same choice as fs_sample's, or fs_sample_packed's).  -1 for an invalid
 * shape. */
FS_API int32_t fs_selected_config(int32_t B, int32_t D, int32_t V);
FS_API int32_t fs_selected_config_packed(int32_t B, int32_t D, int32_t V);
FS_API int32_t fs_selected_config_groups(int32_t B, int32_t D, int32_t V, int32_t packed);

/* Profiling of the fused kernel.  fs_profile_enable(capacity) creates
 * 2 * capacity HIP events (outside any sampling call); while enabled, each of
 * the next `capacity` fs_sample / fs_sample_partial / fs_sample_partial_lse
 * calls (and their _packed forms) records one event before and one after its
 * fused-kernel launch, on the caller's stream (the online sampler's chunk
 * launches are not recorded).
 * fs_profile_read waits for the recorded events, returns the number of timed
 * launches and the sum, minimum and maximum of their durations in
 * milliseconds (any output may be NULL), and re-arms the recorder.
 * fs_profile_enable(0) destroys the events.  Not for concurrent callers. */
FS_API fs_status fs_profile_enable(int32_t capacity);
FS_API fs_status fs_profile_read(int32_t* launches, double* total_ms, double* min_ms,
                                 double* max_ms);

FS_API const char* fs_status_string(fs_status s);
FS_API const char* fs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHSAMPLE_H */
