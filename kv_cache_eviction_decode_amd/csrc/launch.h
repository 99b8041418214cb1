// Internal launchers: host-side entry into each kernel family. Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

// 1/ln(2): logits are kept in base-2 units so that v_exp_f32 (2^x) is the only
// transcendental on the path.
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const void* K;       // [G][k][d] cache rows (or [G][len][d] full cache)
  const void* V;
  float* score;        // [G][k]           (scored mode only)
  int32_t* pos;        // [G][k]           (scored mode only)
  void* K_w;           // writable aliases of K, V for the new token (scored mode)
  void* V_w;
  const void* q;       // [G][d]
  const void* k_new;   // [G][d]           (scored mode only)
  const void* v_new;   // [G][d]           (scored mode only)
  float* out;          // [G][d] fp32
  int32_t* evicted;    // [G]              (scored mode only)
  const float* k_qparam;  // [G][2][d] key grids (8-bit caches only)
  float* v_qparam;        // [G][k][2] value grids (8-bit caches only)
  int32_t k;           // slot capacity (rows per head in K/V)
  int32_t n_used;      // occupied slots [0, n_used), or full-cache length
  int32_t t;           // position of the new token
  int32_t k_recent;
  int32_t policy;      // h2o_policy
  float c;             // scale * log2(e)
};

// Compute units of the current device (256 on MI355X).
int cu_count();

// Fused H2O decode step: attention over n_used slots + the new token, score
// accumulation, at most one eviction, insert. One workgroup per head.
hipError_t launch_decode(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s);

// Decode step of a cache stored as 8-bit codes (K, V point to the codes).
hipError_t launch_decode_u8(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s);

// Split decode: the occupied slots of every head are cut into `chunks` runs of
// `chunk_len` rows (the last one ragged), each streamed by its own wave; a
// second kernel merges them per head.
struct SplitArgs {
  float* logit;       // [G][k] logits of the step, base-2 units
  float* part_ml;     // [G][cmax][2] per-chunk (max, sum) of the online softmax
  float* part_acc;    // [G][cmax][d] per-chunk unnormalised P.V
  int32_t chunk_len;  // rows per chunk, a multiple of 64
  int32_t chunks;     // ceil(n_used / chunk_len), at least 1
  int32_t cmax;       // chunk capacity per head in the workspace
};
// Chunks of at least 64 rows over at most 8192 slots.
constexpr int kMaxChunks = 128;

hipError_t launch_decode_split(int dtype, int head_dim, int G, const DecodeArgs& a, const SplitArgs& s,
                               hipStream_t st);

// Plain attention of one query over a contiguous cache of n_used rows.
hipError_t launch_fullcache(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s);

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
