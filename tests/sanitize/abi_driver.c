/* Drives every entry point of libflashsample's C ABI through its host-side
 * paths, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * invalid arguments, size queries at extreme values, configuration queries,
 * and calls with valid arguments made only under FS_FAULT_INJECT=launch, so
 * that nothing is ever launched (the pointers below are fake and are never
 * dereferenced).  Exits non-zero on the first unexpected status. */
#define _POSIX_C_SOURCE 200809L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flashsample.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d: %s\n", what, got,
            fs_status_string((fs_status)got), want, fs_last_error());
    ++failures;
  }
  (void)strlen(fs_last_error());
}

#define A ((void*)(uintptr_t)0x10000)
#define WS ((void*)(uintptr_t)0x20000)
#define F ((float*)(uintptr_t)0x10000)
#define I ((int32_t*)(uintptr_t)0x10000)
#define DB ((double*)(uintptr_t)0x10000)

int main(void) {
  const size_t big = (size_t)1 << 40;
  int32_t cuts[3] = {0, 512, 1000};
  int32_t bad_cuts[3] = {0, 600, 600};
  int32_t odd_cuts[3] = {0, 500, 1000};  /* 500 is not a multiple of 16 */

  /* size queries over extreme arguments: no overflow, zero when invalid */
  const int32_t Bs[] = {-1, 0, 1, 65535, 1 << 20, 1 << 29, INT32_MAX};
  const int32_t Ds[] = {-8, 0, 7, 8, 4096, 32768, INT32_MAX - 7};
  const int32_t Vs[] = {-1, 0, 1, 16032, 128256, INT32_MAX};
  for (size_t b = 0; b < sizeof Bs / sizeof *Bs; ++b)
    for (size_t d = 0; d < sizeof Ds / sizeof *Ds; ++d)
      for (size_t v = 0; v < sizeof Vs / sizeof *Vs; ++v) {
        (void)fs_workspace_bytes(Bs[b], Ds[d], Vs[v]);
        (void)fs_unfused_workspace_bytes(Bs[b], Ds[d], Vs[v]);
        (void)fs_online_workspace_bytes(Bs[b], Ds[d], Vs[v], 8);
        (void)fs_packed_weights_bytes(Vs[v], Ds[d], 3);
        (void)fs_online_bounds_workspace_bytes(Vs[v], 65536);
        (void)fs_selected_config(Bs[b], Ds[d], Vs[v]);
        (void)fs_selected_config_packed(Bs[b], Ds[d], Vs[v]);
      }
  if (fs_unfused_workspace_bytes(1 << 29, 8, 64) < ((size_t)2 << 29) * 64 * 4) {
    fprintf(stderr, "unfused workspace size wrapped\n");
    ++failures;
  }

  /* configuration table */
  const int32_t n = fs_num_configs();
  for (int32_t i = -1; i <= n; ++i) (void)fs_config_name(i);
  expect("force -2", fs_force_config(-2), FS_ERR_INVALID_ARG);
  expect("force n", fs_force_config(n), FS_ERR_INVALID_ARG);
  expect("force 0", fs_force_config(0), FS_OK);
  expect("force -1", fs_force_config(-1), FS_OK);
  for (int s = -1; s <= 5; ++s) (void)fs_status_string((fs_status)s);

  /* invalid arguments, one entry point at a time */
  expect("sample D=7", fs_sample(A, A, 4, 7, 1000, 0, F, 1, 2, I, F, WS, big, NULL), FS_ERR_INVALID_ARG);
  expect("sample V=0", fs_sample(A, A, 4, 256, 0, 0, F, 1, 2, I, F, WS, big, NULL), FS_ERR_INVALID_ARG);
  expect("sample off", fs_sample(A, A, 4, 256, 1000, INT32_MAX - 10, F, 1, 2, I, F, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("sample null", fs_sample(NULL, A, 4, 256, 1000, 0, F, 1, 2, I, F, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("sample ws", fs_sample(A, A, 4, 256, 1000, 0, F, 1, 2, I, F, WS, 16, NULL), FS_ERR_WORKSPACE);
  expect("sample B huge", fs_sample(A, A, INT32_MAX, 256, 1000, 0, F, 1, 2, I, F, WS, (size_t)-1, NULL),
         FS_ERR_UNSUPPORTED);
  expect("sample B=0", fs_sample(NULL, NULL, 0, 256, 1000, 0, NULL, 1, 2, NULL, NULL, NULL, 0, NULL),
         FS_OK);
  expect("packed D=72", fs_sample_packed(A, A, 4, 72, 1000, 0, F, 1, 2, I, F, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("noalloc large", fs_sample_packed_noalloc(A, A, 2048, 256, 200000, 0, F, 1, 2, I, F, NULL),
         FS_ERR_WORKSPACE);
  expect("partial_lse null lse",
         fs_sample_partial_lse(A, A, 4, 256, 1000, 0, F, 1, 2, F, I, NULL, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("unfused B", fs_sample_unfused(A, A, 65536, 256, 1000, 0, F, 1, 2, I, F, WS, big, NULL),
         FS_ERR_UNSUPPORTED);
  expect("merge P=0", fs_merge(F, I, 0, 4, I, F, NULL), FS_ERR_INVALID_ARG);
  expect("merge P*B", fs_merge(F, I, 1 << 20, 1 << 21, I, F, NULL), FS_ERR_INVALID_ARG);
  expect("merge_lse align", fs_merge_lse(F, I, (float*)((char*)F + 2), 2, 4, F, 1, 2, I, F, F, NULL),
         FS_ERR_INVALID_ARG);
  expect("pack D", fs_pack_weights(A, 1000, 72, 0, A, big, NULL), FS_ERR_INVALID_ARG);
  expect("pack bytes", fs_pack_weights(A, 1000, 256, 0, A, 16, NULL), FS_ERR_WORKSPACE);
  expect("bounds cuts", fs_online_bounds(A, 1000, 256, bad_cuts, 2, DB, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("bounds n", fs_online_bounds(A, 1000, 256, cuts, 70000, DB, WS, big, NULL), FS_ERR_INVALID_ARG);
  expect("online D", fs_sample_online(A, A, 4, 32776, 1000, 0, F, 1, 2, cuts, 2, DB, I, F, I, WS, big,
                                      NULL), FS_ERR_UNSUPPORTED);
  expect("online packed cut", fs_sample_online_packed(A, A, 4, 256, 1000, 0, F, 1, 2, odd_cuts, 2, DB, I,
                                                      F, I, WS, big, NULL), FS_ERR_INVALID_ARG);
  for (int packed = 0; packed <= 1; ++packed)
    for (int i = 0; i < 7; ++i) (void)fs_selected_config_groups(Bs[i], 4096, 128256, packed);
  expect("groups cuts", fs_sample_groups_lse(A, A, 4, 256, 1000, 0, F, 1, 2, bad_cuts, 2, F, I, F, WS, big,
                                             NULL), FS_ERR_INVALID_ARG);
  expect("groups n", fs_sample_groups_lse(A, A, 4, 256, 1000, 0, F, 1, 2, cuts, 65, F, I, F, WS, big, NULL),
         FS_ERR_INVALID_ARG);
  expect("groups packed cut", fs_sample_groups_lse_packed(A, A, 4, 256, 1000, 0, F, 1, 2, odd_cuts, 2, F, I,
                                                          F, WS, big, NULL), FS_ERR_INVALID_ARG);
  expect("groups ws", fs_sample_groups_lse(A, A, 4, 256, 1000, 0, F, 1, 2, cuts, 2, F, I, F, WS, 16, NULL),
         FS_ERR_WORKSPACE);
  expect("noise n", fs_debug_noise(0, 0, 0, 0, -1, (uint32_t*)I, F, NULL), FS_ERR_INVALID_ARG);
  expect("noise range", fs_debug_noise(0, 0, 0, UINT32_MAX - 2, 5, (uint32_t*)I, F, NULL),
         FS_ERR_INVALID_ARG);
  expect("gumbel null", fs_debug_gumbel(NULL, 5, F, NULL), FS_ERR_INVALID_ARG);
  expect("device -1", fs_device_info(-1, NULL, NULL), FS_ERR_INVALID_ARG);
  expect("profile -1", fs_profile_enable(-1), FS_ERR_INVALID_ARG);

  /* valid arguments, launches refused by the injection hook */
  setenv("FS_FAULT_INJECT", "launch", 1);
  expect("inj sample", fs_sample(A, A, 4, 256, 1000, 0, F, 1, 2, I, F, WS, big, NULL), FS_ERR_HIP);
  expect("inj sample B=300", fs_sample(A, A, 300, 256, 3001, 5, F, 1, 2, I, F, WS, big, NULL), FS_ERR_HIP);
  expect("inj partial", fs_sample_partial(A, A, 4, 256, 1000, 3, F, 1, 2, F, I, WS, big, NULL), FS_ERR_HIP);
  expect("inj packed", fs_sample_packed(A, A, 32, 4096, 128256, 0, F, 1, 2, I, F, WS, big, NULL),
         FS_ERR_HIP);
  expect("inj noalloc", fs_sample_packed_noalloc(A, A, 4, 256, 1000, 0, F, 1, 2, I, F, NULL), FS_ERR_HIP);
  expect("inj partial_lse",
         fs_sample_partial_lse(A, A, 4, 256, 1000, 0, F, 1, 2, F, I, F, WS, big, NULL), FS_ERR_HIP);
  expect("inj partial_lse_packed",
         fs_sample_partial_lse_packed(A, A, 4, 256, 1000, 0, F, 1, 2, F, I, F, WS, big, NULL), FS_ERR_HIP);
  expect("inj groups", fs_sample_groups_lse(A, A, 4, 256, 1000, 0, F, 1, 2, cuts, 2, F, I, F, WS, big, NULL),
         FS_ERR_HIP);
  expect("inj groups packed", fs_sample_groups_lse_packed(A, A, 4, 256, 1000, 0, F, 1, 2, cuts, 2, F, I, F, WS,
                                                          big, NULL), FS_ERR_HIP);
  expect("inj unfused", fs_sample_unfused(A, A, 4, 256, 1000, 0, F, 1, 2, I, F, WS, big, NULL), FS_ERR_HIP);
  expect("inj merge", fs_merge(F, I, 3, 4, I, F, NULL), FS_ERR_HIP);
  expect("inj merge_lse", fs_merge_lse(F, I, F, 3, 4, F, 1, 2, I, F, F, NULL), FS_ERR_HIP);
  expect("inj pack", fs_pack_weights(A, 1000, 256, 1, A, big, NULL), FS_ERR_HIP);
  expect("inj bounds", fs_online_bounds(A, 1000, 256, cuts, 2, DB, WS, big, NULL), FS_ERR_HIP);
  expect("inj bounds packed", fs_online_bounds_packed(A, 1000, 256, 2, cuts, 2, DB, WS, big, NULL), FS_ERR_HIP);
  expect("inj online", fs_sample_online(A, A, 4, 256, 1000, 0, F, 1, 2, cuts, 2, DB, I, F, I, WS, big, NULL),
         FS_ERR_HIP);
  expect("inj noise", fs_debug_noise(0, 0, 0, 0, 16, (uint32_t*)I, F, NULL), FS_ERR_HIP);
  expect("inj gumbel", fs_debug_gumbel((const uint32_t*)I, 16, F, NULL), FS_ERR_HIP);
  unsetenv("FS_FAULT_INJECT");

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("abi driver: all host paths ran clean\n");
  return 0;
}
