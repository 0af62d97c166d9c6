/*
 * oracle.c -- plain, slow CPU oracle for exact Gumbel-Max sampling fused into
 * the LM-head matmul ("FlashSampling: Fast and Memory-Efficient Exact
 * Sampling").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it and shares no source with it: the Philox generator, the
 * uniform/Gumbel maps, the logits and the comparator below are written here
 * a second time, independently of the HIP kernels.
 *
 * What it computes is the plain definition the method is proved to reach
 * exactly (wiki summary page, "Key claims": argmax over logits plus Gumbel
 * noise decomposes over any partition of the vocabulary, so the tiled kernel
 * returns the same maximiser as one global argmax; arXiv abstract page: the
 * sampler is exact, not approximate):
 *
 *   1. full logits  z[b][v] = sum_d h[b][d] * W[v][d]            (no bias)
 *   2. scaled score s = z * (1/T[b])   (wiki summary, "Method", step 3 of
 *      the four-op decode step: temperature scaling)
 *   3. perturbed    s += g,  g = -log(-log u),  u from a counter-based
 *      generator keyed on (seed, step, row, global vocab index) -- the pages
 *      say only that each element of the tile gets its own Gumbel draw from
 *      the tile's RNG state ("Method"); the generator is Philox-4x32-10
 *      (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *      1, 2, 3", SC'11)
 *   4. one global argmax per row; ties go to the smaller global index.
 *
 * Precision: every dot product is summed in fp64 (bf16 -> fp64 is exact, each
 * product is exact) in increasing d and rounded once to fp32; the Gumbel
 * value is evaluated in fp64 and rounded once to fp32; the temperature scale
 * and the noise add are separate fp32 operations (compile with
 * -ffp-contract=off so that no fused multiply-add is formed).
 *
 * Parallelism: OpenMP over independent outputs only (rows or seeds); no
 * output depends on the thread count or the schedule.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

/* Threads an OpenMP region of the oracle will use. */
ORACLE_EXPORT int oracle_max_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------------- */
/* Philox-4x32-10 (SC'11 paper, section 5: the Philox round is two 32x32->64
 * multiplications by fixed odd constants whose halves are permuted and xored
 * with the other counter words and the round key; the key is bumped by the
 * Weyl increments between rounds).                                         */
/* ---------------------------------------------------------------------- */
static const uint32_t PHILOX_MUL_A = 0xD2511F53u; /* multiplies word 0 */
static const uint32_t PHILOX_MUL_B = 0xCD9E8D57u; /* multiplies word 2 */
static const uint32_t PHILOX_WEYL_0 = 0x9E3779B9u; /* golden ratio */
static const uint32_t PHILOX_WEYL_1 = 0xBB67AE85u; /* sqrt(3) - 1 */

ORACLE_EXPORT void oracle_philox4x32_10(const uint32_t ctr_in[4],
                                        const uint32_t key_in[2],
                                        uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { /* key schedule: bump before every round but the first */
      k0 += PHILOX_WEYL_0;
      k1 += PHILOX_WEYL_1;
    }
    uint64_t prod_a = (uint64_t)PHILOX_MUL_A * (uint64_t)c0;
    uint64_t prod_b = (uint64_t)PHILOX_MUL_B * (uint64_t)c2;
    uint32_t hi_a = (uint32_t)(prod_a >> 32), lo_a = (uint32_t)prod_a;
    uint32_t hi_b = (uint32_t)(prod_b >> 32), lo_b = (uint32_t)prod_b;
    uint32_t n0 = hi_b ^ c1 ^ k0;
    uint32_t n1 = lo_b;
    uint32_t n2 = hi_a ^ c3 ^ k1;
    uint32_t n3 = lo_a;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Raw 32-bit noise word for (seed, step, row, global vocab index gv).
 * Counter = (gv / 4, row, step low word, step high word); key = (seed low
 * word, seed high word); the element takes output word gv mod 4, so one
 * generator call covers four consecutive vocabulary ids.  Keying on the
 * global index makes the noise field independent of how V is tiled or
 * sharded (wiki summary, "Method": per-rank shards use the same per-element
 * draw as an unsharded run).                                               */
ORACLE_EXPORT uint32_t oracle_noise_bits(uint64_t seed, uint64_t step,
                                         uint32_t row, uint32_t gv) {
  uint32_t ctr[4] = {gv >> 2, row, (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return out[gv & 3u];
}

/* Uniform in the open interval (0,1): the midpoint of the word's cell of
 * width 2^-32, u = (x + 1/2) * 2^-32.  All 32 bits of the word count, so two
 * ids share a noise value only when their words are equal (probability
 * 2^-32 per pair): with equal logits the largest score is then tied with
 * probability about V * 2^-33, and the sampler stays exact up to that
 * granularity (wiki summary, "Key claims": the samples follow the
 * categorical distribution with no approximation).  Exact in fp64 (33
 * significant bits); never 0 or 1, so the Gumbel value below is finite.    */
ORACLE_EXPORT double oracle_uniform(uint32_t bits) {
  return ((double)bits + 0.5) * 0x1p-32;
}

/* Standard Gumbel draw by inversion of its CDF exp(-exp(-g)):
 * g = -log(-log u), evaluated in fp64 and rounded once to fp32.            */
ORACLE_EXPORT float oracle_gumbel(uint32_t bits) {
  double u = oracle_uniform(bits);
  double g = -log(-log(u));
  return (float)g;
}

/* Bulk forms of the three maps above, one output per input element.      */
ORACLE_EXPORT void oracle_noise_bits_range(uint64_t seed, uint64_t step,
                                           uint32_t row, uint32_t gv0, int64_t n,
                                           uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = oracle_noise_bits(seed, step, row, gv0 + (uint32_t)i);
}

ORACLE_EXPORT void oracle_uniform_array(const uint32_t* bits, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_uniform(bits[i]);
}

ORACLE_EXPORT void oracle_gumbel_array(const uint32_t* bits, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_gumbel(bits[i]);
}

/* ---------------------------------------------------------------------- */
/* Logits                                                                   */
/* ---------------------------------------------------------------------- */
static double bf16_to_double(uint16_t x) {
  uint32_t w = (uint32_t)x << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* One logit z = sum_d h[d] * W[d], fp64 in increasing d, rounded once.    */
ORACLE_EXPORT float oracle_logit(const uint16_t* h_row, const uint16_t* w_row,
                                 int32_t D) {
  double acc = 0.0;
  for (int32_t d = 0; d < D; ++d)
    acc += bf16_to_double(h_row[d]) * bf16_to_double(w_row[d]);
  return (float)acc;
}

/* Full fp32 logits z[b][v] for b < B, v < V (row-major B x V).            */
ORACLE_EXPORT void oracle_logits(const uint16_t* h, const uint16_t* W,
                                 int32_t B, int32_t D, int32_t V, float* z) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t b = 0; b < B; ++b)
    for (int32_t v = 0; v < V; ++v)
      z[(size_t)b * V + v] = oracle_logit(h + (size_t)b * D, W + (size_t)v * D, D);
}

/* ---------------------------------------------------------------------- */
/* Scores and the global argmax                                             */
/* ---------------------------------------------------------------------- */
/* A row is greedy when its temperature is not a positive number (0, -0,
 * negative or NaN): the T -> 0 limit of the sampler is the plain argmax of
 * the logits, so such rows take s = z with no scaling and no noise.       */
static int is_greedy(float T) { return !(T > 0.0f); }

static float score(float z, float T, float inv_T, uint64_t seed, uint64_t step,
                   uint32_t row, uint32_t gv) {
  if (is_greedy(T)) return z;
  float scaled = z * inv_T;                                 /* fp32 multiply */
  float g = oracle_gumbel(oracle_noise_bits(seed, step, row, gv));
  return scaled + g;                                        /* fp32 add */
}

/* Perturbed score of one element, for checks on a single (row, id).       */
ORACLE_EXPORT float oracle_score(float z, float T, uint64_t seed, uint64_t step,
                                 uint32_t row, uint32_t gv) {
  float inv_T = is_greedy(T) ? 1.0f : 1.0f / T;
  return score(z, T, inv_T, seed, step, row, gv);
}

typedef struct {
  float best;
  int32_t best_id;
  float second; /* largest score among the other ids */
} running_max;

static void rm_init(running_max* r) {
  r->best = -INFINITY;
  r->best_id = -1;
  r->second = -INFINITY;
}

/* Elements arrive in increasing global id, so a strict '>' keeps the
 * smaller id on a tie.                                                     */
static void rm_push(running_max* r, float s, int32_t gv) {
  if (r->best_id < 0 || s > r->best) {
    if (r->best_id >= 0) r->second = r->best;
    r->best = s;
    r->best_id = gv;
  } else if (s > r->second) {
    r->second = s;
  }
}

/* Sample the listed rows (rows == NULL: rows 0..n_rows-1) of a decode step.
 * h is B x D and W is V x D (bf16 bits, row-major); row r of the batch uses
 * noise key (seed, step, r) and its vocabulary ids are vocab_offset + v.
 * Outputs per listed row: sampled global id, winning perturbed score, and
 * the gap between the winner and the runner-up.                            */
ORACLE_EXPORT void oracle_sample(const uint16_t* h, const uint16_t* W,
                                 int32_t D, int32_t V, int32_t vocab_offset,
                                 const float* T, uint64_t seed, uint64_t step,
                                 const int32_t* rows, int32_t n_rows,
                                 int32_t* out_id, float* out_val,
                                 float* out_gap) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t b = rows ? rows[i] : i;
    float Tb = T[b];
    float inv_T = is_greedy(Tb) ? 1.0f : 1.0f / Tb;
    running_max r;
    rm_init(&r);
    for (int32_t v = 0; v < V; ++v) {
      float z = oracle_logit(h + (size_t)b * D, W + (size_t)v * D, D);
      int32_t gv = vocab_offset + v;
      rm_push(&r, score(z, Tb, inv_T, seed, step, (uint32_t)b, (uint32_t)gv), gv);
    }
    out_id[i] = r.best_id;
    out_val[i] = r.best;
    out_gap[i] = r.best - r.second;
  }
}

/* Same, from precomputed fp32 logits: z is n_rows x V and T has n_rows
 * entries, one per listed row; rows[i] (or i) is that row's batch position,
 * which keys its noise.  Repeated for n_seeds consecutive seeds seed0,
 * seed0+1, ...; output index is [seed][row].  Used for distribution checks,
 * where the logits stay fixed and only the noise changes.                  */
ORACLE_EXPORT void oracle_sample_logits(const float* z, int32_t V,
                                        int32_t vocab_offset, const float* T,
                                        uint64_t seed0, int32_t n_seeds,
                                        uint64_t step, const int32_t* rows,
                                        int32_t n_rows, int32_t* out_id,
                                        float* out_val, float* out_gap) {
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t job = 0; job < (int64_t)n_seeds * n_rows; ++job) {
    int32_t si = (int32_t)(job / n_rows), i = (int32_t)(job % n_rows);
    int32_t b = rows ? rows[i] : i;
    float Tb = T[i];
    float inv_T = is_greedy(Tb) ? 1.0f : 1.0f / Tb;
    uint64_t seed = seed0 + (uint64_t)si;
    running_max r;
    rm_init(&r);
    for (int32_t v = 0; v < V; ++v) {
      int32_t gv = vocab_offset + v;
      rm_push(&r, score(z[(size_t)i * V + v], Tb, inv_T, seed, step, (uint32_t)b,
                        (uint32_t)gv), gv);
    }
    out_id[job] = r.best_id;
    if (out_val) out_val[job] = r.best;
    if (out_gap) out_gap[job] = r.best - r.second;
  }
}

/* ---------------------------------------------------------------------- */
/* Merge of per-part (max, argmax) pairs                                    */
/* ---------------------------------------------------------------------- */
/* Partials are P x B, part-major: (val[p*B + b], id[p*B + b]).  Per row the
 * winner is the largest value, and among equal values the smallest id:
 * this is the cross-part argmax that makes per-tile and per-rank maximisers
 * reproduce the global one (wiki summary, "Method").                        */
ORACLE_EXPORT void oracle_merge(const float* val, const int32_t* id, int32_t P,
                                int32_t B, int32_t* out_id, float* out_val) {
  for (int32_t b = 0; b < B; ++b) {
    float best = val[b];
    int32_t best_id = id[b];
    for (int32_t p = 1; p < P; ++p) {
      float v = val[(size_t)p * B + b];
      int32_t i = id[(size_t)p * B + b];
      if (v > best || (v == best && i < best_id)) {
        best = v;
        best_id = i;
      }
    }
    out_id[b] = best_id;
    out_val[b] = best;
  }
}

/* ---------------------------------------------------------------------- */
/* Grouped (hierarchical) sampler                                           */
/* ---------------------------------------------------------------------- */
/* The categorical distribution factorises over any partition of the
 * vocabulary into groups G: P(i) = P(G) * P(i | G), with P(G) proportional
 * to exp(LSE_G), LSE_G = log sum_{i in G} exp(z_i / T) (arXiv abstract page
 * and wiki summary, "Key claims": grouped variants for online and
 * tensor-parallel settings are exact by this hierarchical factorisation).
 * The pages give no formulas; the reading built here:
 *   - a group's own sample is its Gumbel-max winner over the token noise
 *     field above (oracle_sample on the group's slice), distributed as
 *     P(i | G);
 *   - the group is chosen by a second Gumbel-max, argmax_G (LSE_G + gamma_G),
 *     with gamma_G a standard Gumbel draw independent of the token noise;
 *   - the output is the chosen group's sample, plus the total
 *     log-sum-exp over the groups (the normaliser of the whole row).
 * Greedy rows (T not > 0) have a point-mass distribution: LSE_G is the
 * group's largest logit and the group choice takes no noise, which selects
 * the group holding the global argmax.                                     */

/* Gumbel draw of group p for batch row `row`: the token generator with the
 * same key, on counter (2^31 | p, row, step low, step high), output word 0.
 * Token counters have word 0 = gv / 4 < 2^29, so the two streams never
 * share a counter.                                                         */
ORACLE_EXPORT float oracle_group_gumbel(uint64_t seed, uint64_t step, uint32_t row,
                                        uint32_t p) {
  uint32_t ctr[4] = {0x80000000u | p, row, (uint32_t)step, (uint32_t)(step >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  return oracle_gumbel(out[0]);
}

/* As oracle_sample, plus per listed row the log-sum-exp of the slice's
 * scaled logits, log sum_v exp(z_v * (1/T)) with the fp32 reciprocal of
 * T, evaluated in fp64 around the slice maximum and rounded once to fp32;
 * for greedy rows the slice's largest logit.                              */
ORACLE_EXPORT void oracle_sample_lse(const uint16_t* h, const uint16_t* W, int32_t D,
                                     int32_t V, int32_t vocab_offset, const float* T,
                                     uint64_t seed, uint64_t step, const int32_t* rows,
                                     int32_t n_rows, int32_t* out_id, float* out_val,
                                     float* out_gap, float* out_lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t b = rows ? rows[i] : i;
    float Tb = T[b];
    int greedy = is_greedy(Tb);
    float inv_T = greedy ? 1.0f : 1.0f / Tb;
    running_max r;
    rm_init(&r);
    double zmax = -INFINITY;
    double* scaled = (double*)malloc(sizeof(double) * (size_t)V);
    for (int32_t v = 0; v < V; ++v) {
      float z = oracle_logit(h + (size_t)b * D, W + (size_t)v * D, D);
      int32_t gv = vocab_offset + v;
      rm_push(&r, score(z, Tb, inv_T, seed, step, (uint32_t)b, (uint32_t)gv), gv);
      scaled[v] = greedy ? (double)z : (double)z * (double)inv_T;
      if (scaled[v] > zmax) zmax = scaled[v];
    }
    double lse = zmax;
    if (!greedy) {
      double sum = 0.0;
      for (int32_t v = 0; v < V; ++v) sum += exp(scaled[v] - zmax);
      lse = zmax + log(sum);
    }
    free(scaled);
    out_id[i] = r.best_id;
    out_val[i] = r.best;
    out_gap[i] = r.best - r.second;
    out_lse[i] = (float)lse;
  }
}

/* Grouped merge.  Partials are P x B, part-major (val, id, lse), group p in
 * slot p.  Per row b: the group key is lse_p + gamma_p, an fp32 add of the
 * fp32 group draw (greedy rows: lse_p alone); the largest key wins, ties to
 * the smaller p.  Outputs the winner's (id, val), the total log-sum-exp
 * log sum_p exp(lse_p) (fp64 around the maximum, rounded once; greedy rows:
 * the largest lse_p) and the gap between the two largest keys.            */
ORACLE_EXPORT void oracle_merge_lse(const float* val, const int32_t* id, const float* lse,
                                    int32_t P, int32_t B, const float* T, uint64_t seed,
                                    uint64_t step, int32_t* out_id, float* out_val,
                                    float* out_lse, float* out_gap) {
  for (int32_t b = 0; b < B; ++b) {
    int greedy = is_greedy(T[b]);
    int32_t best_p = -1;
    float best_key = -INFINITY, second_key = -INFINITY;
    double lmax = -INFINITY;
    for (int32_t p = 0; p < P; ++p) {
      float l = lse[(size_t)p * B + b];
      float key = greedy ? l : l + oracle_group_gumbel(seed, step, (uint32_t)b, (uint32_t)p);
      if (best_p < 0 || key > best_key) {
        if (best_p >= 0) second_key = best_key;
        best_key = key;
        best_p = p;
      } else if (key > second_key) {
        second_key = key;
      }
      if ((double)l > lmax) lmax = (double)l;
    }
    double total = lmax;
    if (!greedy) {
      double sum = 0.0;
      for (int32_t p = 0; p < P; ++p) sum += exp((double)lse[(size_t)p * B + b] - lmax);
      total = lmax + log(sum);
    }
    out_id[b] = id[(size_t)best_p * B + b];
    out_val[b] = val[(size_t)best_p * B + b];
    out_lse[b] = (float)total;
    out_gap[b] = best_key - second_key;
  }
}

/* Log-sum-exp of fixed fp32 logits, one per row of z (R x V), with the same
 * scaling and evaluation as oracle_sample_lse.                            */
ORACLE_EXPORT void oracle_lse_logits(const float* z, int32_t V, const float* T, int32_t R,
                                     float* out_lse) {
  for (int32_t i = 0; i < R; ++i) {
    int greedy = is_greedy(T[i]);
    float inv_T = greedy ? 1.0f : 1.0f / T[i];
    double zmax = -INFINITY;
    for (int32_t v = 0; v < V; ++v) {
      double s = greedy ? (double)z[(size_t)i * V + v] : (double)z[(size_t)i * V + v] * (double)inv_T;
      if (s > zmax) zmax = s;
    }
    double lse = zmax;
    if (!greedy) {
      double sum = 0.0;
      for (int32_t v = 0; v < V; ++v)
        sum += exp((double)z[(size_t)i * V + v] * (double)inv_T - zmax);
      lse = zmax + log(sum);
    }
    out_lse[i] = (float)lse;
  }
}

/* ---------------------------------------------------------------------- */
/* Online (chunked) sampler with early finalisation                         */
/* ---------------------------------------------------------------------- */
/* The vocabulary arrives as consecutive chunks; the running (max, argmax)
 * is the Gumbel-max over the chunks seen so far, and the sample may be
 * finalised as soon as no later chunk can overtake it (wiki summary,
 * "Method": the streaming sampler of the online setting).  The pages give
 * no bound; the reading built here:
 *   - a later logit obeys z = h . W_v <= |h| * R, R the largest row norm of
 *     the later chunks (Cauchy-Schwarz);
 *   - a noise value is at most g_max, the largest value of the Gumbel map,
 *     taken at the top word: -log(-log(1 - 2^-33));
 *   - row b is final after chunk c when its running best exceeds
 *     (|h_b| * R_c * (1/T) + g_max) * (1 + 2^-8) (greedy rows: |h_b| * R_c *
 *     (1 + 2^-8), no scaling and no noise).  The factor 1 + 2^-8 is a safety
 *     margin for rounding: fp32 logits, scores and norms stay below the bound.
 * The samples are those of oracle_sample over the whole vocabulary, whatever
 * the chunks; this function also reports, per row, how many chunks were
 * needed.                                                                  */
ORACLE_EXPORT double oracle_gumbel_max(void) { return -log(-log(1.0 - ldexp(1.0, -33))); }

/* Euclidean norm of a bf16 row, fp64.                                      */
static double row_norm(const uint16_t* x, int32_t D) {
  double s = 0.0;
  for (int32_t d = 0; d < D; ++d) {
    double v = bf16_to_double(x[d]);
    s += v * v;
  }
  return sqrt(s);
}

/* Largest row norm of W (V x D), fp64.                                     */
ORACLE_EXPORT double oracle_max_row_norm(const uint16_t* W, int32_t V, int32_t D) {
  double m = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    double n = row_norm(W + (size_t)v * D, D);
    if (n > m) m = n;
  }
  return m;
}

/* cuts[0] = 0 < cuts[1] < ... < cuts[n_chunks] = V delimit the chunks of W
 * (V x D).  Per listed row: sampled id, winning score, chunks processed.   */
ORACLE_EXPORT void oracle_sample_online(const uint16_t* h, const uint16_t* W, int32_t D,
                                        int32_t vocab_offset, const int32_t* cuts,
                                        int32_t n_chunks, const float* T, uint64_t seed,
                                        uint64_t step, const int32_t* rows, int32_t n_rows,
                                        int32_t* out_id, float* out_val,
                                        int32_t* out_chunks) {
  const double margin = 1.0 + ldexp(1.0, -8);
  const double g_max = oracle_gumbel_max();
  /* later[c]: the largest row norm in chunks c+1 .. n_chunks-1 (0 if none) */
  double* later = (double*)malloc(sizeof(double) * (size_t)n_chunks);
  double m = 0.0;
  for (int32_t c = n_chunks - 1; c >= 0; --c) {
    later[c] = m;
    double mc = oracle_max_row_norm(W + (size_t)cuts[c] * D, cuts[c + 1] - cuts[c], D);
    if (mc > m) m = mc;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    int32_t b = rows ? rows[i] : i;
    float Tb = T[b];
    int greedy = is_greedy(Tb);
    float inv_T = greedy ? 1.0f : 1.0f / Tb;
    double hn = row_norm(h + (size_t)b * D, D);
    running_max r;
    rm_init(&r);
    int32_t used = n_chunks;
    for (int32_t c = 0; c < n_chunks; ++c) {
      for (int32_t v = cuts[c]; v < cuts[c + 1]; ++v) {
        float z = oracle_logit(h + (size_t)b * D, W + (size_t)v * D, D);
        int32_t gv = vocab_offset + v;
        rm_push(&r, score(z, Tb, inv_T, seed, step, (uint32_t)b, (uint32_t)gv), gv);
      }
      if (c == n_chunks - 1) break;
      double bound = greedy ? hn * later[c] * margin
                            : (hn * later[c] * (double)inv_T + g_max) * margin;
      if ((double)r.best > bound) {
        used = c + 1;
        break;
      }
    }
    out_id[i] = r.best_id;
    out_val[i] = r.best;
    out_chunks[i] = used;
  }
  free(later);
}

/* Threads later OpenMP regions of the oracle use (n <= 0: the default).   */
ORACLE_EXPORT void oracle_set_threads(int n) {
  omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
}
