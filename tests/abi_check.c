/* A plain C99 caller of the library: checks that include/h2o.h is a C header
 * and that the host-side paths of the C ABI (sizes, argument validation,
 * state checks, error messages) work without a GPU. Built and run by
 * test_abi_c.py, and against the host-sanitised build by
 * test_sanitizers_cpu.py. Nothing here reaches a device call. */
#include <stdio.h>
#include <string.h>

#include "h2o.h"

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

static void expect_error(h2o_status got, h2o_status want, const char* needle, const char* what) {
  expect(got == want, what);
  expect(strstr(h2o_last_error(), needle) != NULL, what);
}

int main(void) {
  h2o_cache cache;
  h2o_state state;
  memset(&cache, 0, sizeof cache);

  /* sizes */
  expect(h2o_prefill_workspace_bytes(64, 32, 1024) == (size_t)2 * 64 * 32 * 1024 * 4, "prefill workspace size");
  expect(h2o_prefill_workspace_bytes(1, 1, 1) == 512, "prefill workspace padding");
  expect(h2o_prefill_workspace_bytes(0, 4, 10) == 0, "empty prefill workspace");
  expect(h2o_prefill_workspace_bytes(1, 1, -1) == 0, "negative prompt");
  expect(h2o_decode_workspace_bytes(1, 1, 128, 2048) == (size_t)8192 + 256 + 32 * 128 * 4, "decode workspace size");
  expect(h2o_decode_workspace_bytes(1, 1, 96, 64) == 0, "decode workspace, bad head_dim");
  expect(h2o_decode_workspace_bytes(1, 1, 128, H2O_MAX_SLOTS + 1) == 0, "decode workspace, too many slots");
  expect(strlen(h2o_build_digest()) == 16, "build digest");

  /* cache initialisation: every argument check happens before any launch */
  expect_error(h2o_cache_init(NULL, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.088f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "NULL", "NULL cache rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 100, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "head_dim", "unsupported head_dim rejected");
  expect_error(h2o_cache_init(&cache, 0, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "batch", "empty batch rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, -1, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "k_heavy", "negative k_heavy rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, 0, 0, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "k = k_heavy + k_recent", "empty cache rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, H2O_MAX_SLOTS, 1, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL,
                              NULL, NULL, NULL, NULL), H2O_EINVAL, "exceeds", "too many slots rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, 8, 8, 7, H2O_BF16, 0.1f, NULL, NULL, NULL, NULL, NULL), H2O_EINVAL,
               "policy", "unknown policy rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, 9, 0.1f, NULL, NULL, NULL, NULL,
                              NULL), H2O_EINVAL, "dtype", "unknown dtype rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, -1.f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "scale", "bad scale rejected");
  expect_error(h2o_cache_init(&cache, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL,
                              NULL, NULL), H2O_EINVAL, "non-NULL", "missing buffers rejected");
  expect_error(h2o_cache_init_quant(&cache, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, 5, NULL, NULL,
                                    NULL, NULL, NULL, NULL, NULL), H2O_EINVAL, "code format", "unknown codes rejected");
  expect_error(h2o_cache_init_quant(&cache, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, H2O_QUANT_U4,
                                    NULL, NULL, NULL, NULL, NULL, NULL, NULL), H2O_EINVAL, "k_qparam",
               "missing grids rejected");
  expect(cache.magic == 0, "descriptor untouched by failed inits");

  /* calls on a descriptor h2o_cache_init never filled */
  expect(h2o_decode_step(&cache, NULL, NULL, NULL, NULL, NULL, NULL) == H2O_ESTATE, "uninitialised decode");
  expect(h2o_decode_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL) == H2O_EINVAL, "NULL decode");
  expect(h2o_decode_step_split(&cache, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL) == H2O_ESTATE,
         "uninitialised split decode");
  expect(h2o_decode_step_split_noalloc(&cache, NULL, NULL, NULL, NULL, NULL, 0, NULL) == H2O_ESTATE,
         "uninitialised allocation-free split decode");
  expect(h2o_prefill_select(&cache, NULL, NULL, NULL, 4, NULL, 0, NULL, NULL) == H2O_ESTATE, "uninitialised prefill");
  expect(h2o_cache_state(&cache, &state, NULL, NULL, NULL) == H2O_ESTATE, "uninitialised state");
  expect(h2o_cache_restore(&cache, 3, 0) == H2O_ESTATE, "uninitialised restore");

  /* the allocation-free step refuses a shape beyond its own workspace before any device call */
  {
    h2o_cache big;
    memset(&big, 0, sizeof big);
    big.batch = 8;
    big.heads = 32;
    big.head_dim = 128;
    big.k_heavy = 4096;
    big.k_recent = 4096;
    big.magic = 0x48324F31u;
    expect(h2o_decode_workspace_bytes(8, 32, 128, 8192) > H2O_SPLIT_SCRATCH_BYTES, "big shape exceeds the array");
    expect_error(h2o_decode_step_split_noalloc(&big, NULL, NULL, NULL, NULL, NULL, 0, NULL), H2O_EWORKSPACE,
                 "split-decode workspace", "oversized allocation-free step rejected");
    /* host counters of that descriptor: restore and state touch no device memory without copies */
    expect(h2o_cache_restore(&big, 5000, 7) == H2O_OK, "restore counters");
    expect(h2o_cache_state(&big, &state, NULL, NULL, NULL) == H2O_OK, "state without copies");
    expect(state.t_next == 5000 && state.n_used == 5000 && state.k == 8192 && state.steps == 7, "state counters");
    expect(h2o_cache_restore(&big, -1, 0) == H2O_EINVAL, "negative position rejected");
  }

  /* the comparator's argument checks */
  expect_error(h2o_fullcache_decode(1, 1, 128, H2O_BF16, 0.1f, 0, NULL, NULL, NULL, NULL, NULL), H2O_EINVAL, "len",
               "empty full cache rejected");
  expect(h2o_fullcache_decode(1, 1, 100, H2O_BF16, 0.1f, 4, NULL, NULL, NULL, NULL, NULL) == H2O_EINVAL,
         "full cache head_dim rejected");

  if (failures == 0) printf("abi_check ok\n");
  return failures == 0 ? 0 : 1;
}
