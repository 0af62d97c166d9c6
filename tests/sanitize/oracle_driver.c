/* Drives every function the CPU oracle exports on small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (and OpenMP), and
 * checks the outputs are in range.  Exits non-zero on an inconsistency. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exports (oracle/oracle.c) */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t oracle_noise_bits(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv);
double oracle_uniform(uint32_t bits);
float oracle_gumbel(uint32_t bits);
void oracle_noise_bits_range(uint64_t seed, uint64_t step, uint32_t row, uint32_t gv0, int64_t n,
                             uint32_t* out);
void oracle_uniform_array(const uint32_t* bits, int64_t n, double* out);
void oracle_gumbel_array(const uint32_t* bits, int64_t n, float* out);
float oracle_logit(const uint16_t* h_row, const uint16_t* w_row, int32_t D);
void oracle_logits(const uint16_t* h, const uint16_t* W, int32_t B, int32_t D, int32_t V, float* z);
float oracle_score(float z, float T, uint64_t seed, uint64_t step, uint32_t row, uint32_t gv);
void oracle_sample(const uint16_t* h, const uint16_t* W, int32_t D, int32_t V, int32_t vocab_offset,
                   const float* T, uint64_t seed, uint64_t step, const int32_t* rows, int32_t n_rows,
                   int32_t* out_id, float* out_val, float* out_gap);
void oracle_sample_logits(const float* z, int32_t V, int32_t vocab_offset, const float* T,
                          uint64_t seed0, int32_t n_seeds, uint64_t step, const int32_t* rows,
                          int32_t n_rows, int32_t* out_id, float* out_val, float* out_gap);
void oracle_merge(const float* val, const int32_t* id, int32_t P, int32_t B, int32_t* out_id,
                  float* out_val);
float oracle_group_gumbel(uint64_t seed, uint64_t step, uint32_t row, uint32_t p);
void oracle_sample_lse(const uint16_t* h, const uint16_t* W, int32_t D, int32_t V,
                       int32_t vocab_offset, const float* T, uint64_t seed, uint64_t step,
                       const int32_t* rows, int32_t n_rows, int32_t* out_id, float* out_val,
                       float* out_gap, float* out_lse);
void oracle_merge_lse(const float* val, const int32_t* id, const float* lse, int32_t P, int32_t B,
                      const float* T, uint64_t seed, uint64_t step, int32_t* out_id, float* out_val,
                      float* out_lse, float* out_gap);
void oracle_lse_logits(const float* z, int32_t V, const float* T, int32_t R, float* out_lse);
double oracle_gumbel_max(void);
double oracle_max_row_norm(const uint16_t* W, int32_t V, int32_t D);
void oracle_sample_online(const uint16_t* h, const uint16_t* W, int32_t D, int32_t vocab_offset,
                          const int32_t* cuts, int32_t n_chunks, const float* T, uint64_t seed,
                          uint64_t step, const int32_t* rows, int32_t n_rows, int32_t* out_id,
                          float* out_val, int32_t* out_chunks);
void oracle_set_threads(int n);
int oracle_max_threads(void);

static int bad = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++bad; } } while (0)

static uint16_t bf16(float x) {
  uint32_t w;
  memcpy(&w, &x, 4);
  return (uint16_t)((w + 0x7FFF + ((w >> 16) & 1)) >> 16);
}

int main(void) {
  enum { B = 5, D = 40, V = 97, P = 3 };
  uint16_t* h = malloc(sizeof(uint16_t) * B * D);
  uint16_t* W = malloc(sizeof(uint16_t) * V * D);
  uint32_t s = 12345;
  for (int i = 0; i < B * D; ++i) { s = s * 1664525u + 1013904223u; h[i] = bf16(((int)(s >> 16) - 32768) / 16384.0f); }
  for (int i = 0; i < V * D; ++i) { s = s * 1664525u + 1013904223u; W[i] = bf16(((int)(s >> 16) - 32768) / 300000.0f); }
  float T[B] = {1.0f, 0.5f, 0.0f, -1.0f, 2.0f};

  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out4[4];
  oracle_philox4x32_10(ctr, key, out4);
  uint32_t bits[64];
  oracle_noise_bits_range(~0ull, ~0ull, UINT32_MAX, UINT32_MAX - 63, 64, bits);
  CHECK(bits[63] == oracle_noise_bits(~0ull, ~0ull, UINT32_MAX, UINT32_MAX));
  double u[64];
  float g[64];
  oracle_uniform_array(bits, 64, u);
  oracle_gumbel_array(bits, 64, g);
  for (int i = 0; i < 64; ++i) CHECK(u[i] > 0.0 && u[i] < 1.0 && isfinite(g[i]));
  CHECK(oracle_uniform(0) > 0.0 && oracle_uniform(UINT32_MAX) < 1.0);
  CHECK(isfinite(oracle_gumbel(0)) && isfinite(oracle_gumbel(UINT32_MAX)));
  CHECK(oracle_gumbel_max() > 22.0);

  float z[B * V];
  oracle_logits(h, W, B, D, V, z);
  CHECK(z[7] == oracle_logit(h, W + 7 * D, D));
  (void)oracle_score(z[0], 1.0f, 1, 2, 3, 4);

  int32_t ids[B], rows[2] = {4, 1};
  float val[B], gap[B], lse[B];
  for (int nt = 1; nt <= 3; nt += 2) {
    oracle_set_threads(nt);
    CHECK(oracle_max_threads() >= 1);
    oracle_sample(h, W, D, V, 2147483647 - V, T, 7, 8, NULL, B, ids, val, gap);
    for (int b = 0; b < B; ++b) CHECK(ids[b] >= 2147483647 - V && gap[b] >= 0.0f);
    oracle_sample(h, W, D, V, 0, T, 7, 8, rows, 2, ids, val, gap);
    oracle_sample_lse(h, W, D, V, 5, T, 7, 8, NULL, B, ids, val, gap, lse);
    for (int b = 0; b < B; ++b) CHECK(ids[b] >= 5 && ids[b] < 5 + V);
  }
  oracle_set_threads(0);

  int32_t sids[3 * B];
  float sval[3 * B], sgap[3 * B];
  oracle_sample_logits(z, V, 0, T, 100, 3, 1, NULL, B, sids, sval, sgap);
  oracle_sample_logits(z, V, 0, T, 100, 1, 1, NULL, B, sids, NULL, NULL);

  float pv[P * B], pl[P * B];
  int32_t pi[P * B];
  for (int i = 0; i < P * B; ++i) { pv[i] = (float)(i % 4); pi[i] = 1000 - i; pl[i] = (float)i * 0.1f; }
  float mval[B], mlse[B], mgap[B];
  int32_t mid[B];
  oracle_merge(pv, pi, P, B, mid, mval);
  oracle_merge_lse(pv, pi, pl, P, B, T, 3, 4, mid, mval, mlse, mgap);
  (void)oracle_group_gumbel(3, 4, 5, 0x7FFFFFFF);
  oracle_lse_logits(z, V, T, B, mlse);
  for (int b = 0; b < B; ++b) CHECK(isfinite(mlse[b]));

  CHECK(oracle_max_row_norm(W, V, D) > 0.0);
  int32_t cuts[4] = {0, 10, 50, V}, used[B];
  oracle_sample_online(h, W, D, 0, cuts, 3, T, 7, 8, NULL, B, ids, val, used);
  for (int b = 0; b < B; ++b) CHECK(used[b] >= 1 && used[b] <= 3);

  free(h);
  free(W);
  if (bad) return 1;
  printf("oracle driver: all exports ran clean\n");
  return 0;
}
