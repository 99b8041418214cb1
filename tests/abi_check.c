/* A plain C99 caller of the library: checks that include/h2o.h is a C header
 * and that the host-side paths of the C ABI (sizes, argument validation,
 * error messages) work without a GPU. Built and run by test_abi_c.py. */
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

int main(void) {
  h2o_cache cache;
  memset(&cache, 0, sizeof cache);
  expect(h2o_prefill_workspace_bytes(64, 32, 1024) == (size_t)2 * 64 * 32 * 1024 * 4, "prefill workspace size");
  expect(h2o_prefill_workspace_bytes(0, 4, 10) == 0, "empty prefill workspace");
  expect(h2o_decode_workspace_bytes(1, 1, 128, 2048) == (size_t)8192 + 256 + 32 * 128 * 4, "decode workspace size");
  expect(h2o_cache_init(NULL, 1, 1, 128, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.088f, NULL, NULL, NULL, NULL,
                        NULL) == H2O_EINVAL, "NULL cache rejected");
  expect(strlen(h2o_last_error()) > 0, "error message set");
  expect(h2o_cache_init(&cache, 1, 1, 100, 8, 8, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.1f, NULL, NULL, NULL, NULL,
                        NULL) == H2O_EINVAL, "unsupported head_dim rejected");
  expect(h2o_decode_step(&cache, NULL, NULL, NULL, NULL, NULL, NULL) == H2O_ESTATE, "uninitialised cache rejected");
  if (failures == 0) printf("abi_check ok\n");
  return failures == 0 ? 0 : 1;
}
