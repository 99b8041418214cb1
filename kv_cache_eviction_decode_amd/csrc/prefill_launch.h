// Internal launchers of the prefill kernels (scoring, selection, gather) and
// of the cache clear. Arguments are validated by the C ABI layer first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

struct PrefillArgs {
  const void* Q;   // [G][n][d]
  const void* K;   // [G][n][d]
  const void* V;   // [G][n][d]
  float* lse2;     // [G][n] workspace: per-row log2-sum-exp2 of c*s
  float* colsum;   // [G][n] column sums (workspace or caller buffer)
  void* cK;        // cache tensors [G][k][d], [G][k]
  void* cV;
  float* cscore;
  int32_t* cpos;
  int32_t n;
  int32_t k_heavy, k_recent;
  int32_t policy;  // h2o_policy
  float c;         // scale * log2(e)
  int32_t quant;   // h2o_quant of the cache
  float* kq_param; // [G][2][d] key grids (8-bit caches)
  float* vq_param; // [G][k][2] value grids (8-bit caches)
  int32_t pass1;   // PASS1_* below: how the row normalisers are obtained
  float* out;      // [G][n][d] fp32 prompt attention output (PASS1_ATTENTION)
  float* lse_out;  // [G][n] natural-log row normalisers, optional (PASS1_ATTENTION)
  const float* lse_in;  // [G][n] natural-log row normalisers given by the caller (PASS1_GIVEN)
};

// Pass 1 of the prefill: row normalisers only, normalisers together with the
// prompt's attention output, or normalisers handed in by the caller.
enum : int32_t { PASS1_LSE = 0, PASS1_ATTENTION = 1, PASS1_GIVEN = 2 };

hipError_t launch_prefill(int dtype, int head_dim, int G, const PrefillArgs& a, hipStream_t s);

// pos = -1, score = 0 for G*k slots.
hipError_t launch_cache_clear(float* score, int32_t* pos, int64_t count, hipStream_t s);

}  // namespace h2o
