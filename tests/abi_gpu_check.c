/* The C ABI driven from plain C on the GPU, with no Python or PyTorch: device
 * buffers from hipMalloc, cache init, prefill and decode steps through
 * include/h2o.h, results read back with h2o_cache_state and hipMemcpy.
 * All-zero queries make every attention row uniform, so the expected values
 * are a closed form: the selection is the first k_heavy positions plus the
 * window, every full step evicts t - k_recent, and the output is the mean of
 * the values of the cached positions and the new one (value of position j is
 * j in every channel, exact in bf16). Built and run by test_abi_c.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "h2o.h"

enum { B = 1, H = 2, D = 64, N = 64, KH = 8, KR = 8, K = KH + KR, T = 5 };

static uint16_t bf16(float x) {  /* exact for the small integers used here */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (uint16_t)(u >> 16);
}

#define CHECK_HIP(x) do { if ((x) != hipSuccess) { fprintf(stderr, "HIP error at %s\n", #x); return 1; } } while (0)
#define CHECK_H2O(x) do { if ((x) != H2O_OK) { fprintf(stderr, "%s: %s\n", #x, h2o_last_error()); return 1; } } while (0)

int main(void) {
  const size_t prompt = (size_t)B * H * N * D, row = (size_t)B * H * D, slots = (size_t)B * H * K;
  uint16_t* hq = calloc(prompt, sizeof *hq);
  uint16_t* hk = malloc(prompt * sizeof *hk);
  uint16_t* hv = malloc(prompt * sizeof *hv);
  for (size_t g = 0; g < (size_t)B * H; ++g)
    for (int j = 0; j < N; ++j)
      for (int c = 0; c < D; ++c) {
        hk[(g * N + j) * D + c] = bf16((float)((j + c) % 7) - 3.0f);
        hv[(g * N + j) * D + c] = bf16((float)j);
      }
  void *dQ, *dK, *dV, *cK, *cV, *dq, *dk, *dv, *ws;
  float *score, *out;
  int32_t *pos, *ev;
  const size_t ws_bytes = h2o_prefill_workspace_bytes(B, H, N);
  CHECK_HIP(hipMalloc(&dQ, prompt * 2));
  CHECK_HIP(hipMalloc(&dK, prompt * 2));
  CHECK_HIP(hipMalloc(&dV, prompt * 2));
  CHECK_HIP(hipMalloc(&cK, slots * D * 2));
  CHECK_HIP(hipMalloc(&cV, slots * D * 2));
  CHECK_HIP(hipMalloc((void**)&score, slots * 4));
  CHECK_HIP(hipMalloc((void**)&pos, slots * 4));
  CHECK_HIP(hipMalloc(&dq, row * 2));
  CHECK_HIP(hipMalloc(&dk, row * 2));
  CHECK_HIP(hipMalloc(&dv, row * 2));
  CHECK_HIP(hipMalloc((void**)&out, row * 4));
  CHECK_HIP(hipMalloc((void**)&ev, (size_t)B * H * 4));
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemcpy(dQ, hq, prompt * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dK, hk, prompt * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dV, hv, prompt * 2, hipMemcpyHostToDevice));

  h2o_cache cache;
  CHECK_H2O(h2o_cache_init(&cache, B, H, D, KH, KR, H2O_POLICY_ACCUMULATED, H2O_BF16, 0.125f, cK, cV, score, pos,
                           NULL));
  CHECK_H2O(h2o_prefill_select(&cache, dQ, dK, dV, N, ws, ws_bytes, NULL, NULL));

  int members[B * H][K];
  int32_t hpos[B * H * K];
  h2o_state st;
  CHECK_H2O(h2o_cache_state(&cache, &st, hpos, NULL, NULL));
  int failures = 0;
  if (st.n_used != K || st.t_next != N) ++failures;
  for (int g = 0; g < B * H; ++g)
    for (int s = 0; s < K; ++s) {
      const int want = s < KH ? s : N - KR + (s - KH);
      members[g][s] = hpos[g * K + s];
      if (hpos[g * K + s] != want) ++failures;
    }

  uint16_t* hrow = malloc(row * sizeof *hrow);
  float* hout = malloc(row * sizeof *hout);
  int32_t hev[B * H];
  for (int t = 0; t < T; ++t) {
    const int p = N + t;
    memset(hrow, 0, row * 2);
    CHECK_HIP(hipMemcpy(dq, hrow, row * 2, hipMemcpyHostToDevice));
    for (size_t i = 0; i < row; ++i) hrow[i] = bf16(1.0f);
    CHECK_HIP(hipMemcpy(dk, hrow, row * 2, hipMemcpyHostToDevice));
    for (size_t i = 0; i < row; ++i) hrow[i] = bf16((float)p);
    CHECK_HIP(hipMemcpy(dv, hrow, row * 2, hipMemcpyHostToDevice));
    CHECK_H2O(h2o_decode_step(&cache, dq, dk, dv, out, ev, NULL));
    CHECK_HIP(hipMemcpy(hout, out, row * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(hev, ev, sizeof hev, hipMemcpyDeviceToHost));
    for (int g = 0; g < B * H; ++g) {
      double mean = p;
      for (int s = 0; s < K; ++s) mean += members[g][s];
      mean /= K + 1;
      for (int c = 0; c < D; ++c)
        if (fabs(hout[g * D + c] - mean) > 1e-3 * mean) ++failures;
      if (hev[g] != p - KR) ++failures;
      for (int s = 0; s < K; ++s)
        if (members[g][s] == p - KR) members[g][s] = p;
    }
  }
  CHECK_H2O(h2o_cache_state(&cache, &st, hpos, NULL, NULL));
  for (int g = 0; g < B * H; ++g)
    for (int s = 0; s < K; ++s)
      if (hpos[g * K + s] != members[g][s]) ++failures;
  hipFree(dQ); hipFree(dK); hipFree(dV); hipFree(cK); hipFree(cV); hipFree(score); hipFree(pos);
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(out); hipFree(ev); hipFree(ws);
  free(hq); free(hk); free(hv); free(hrow); free(hout);
  if (failures) {
    fprintf(stderr, "%d mismatches\n", failures);
    return 1;
  }
  printf("abi_gpu_check ok\n");
  return 0;
}
