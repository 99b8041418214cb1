// Internal launchers of the decode kernels. Arguments are
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
  const float* k_qparam;  // [G][2][d] key grids (caches stored as codes only)
  float* v_qparam;        // [G][k][2] value grids (caches stored as codes only)
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

// Decode step of a cache stored as bits-wide codes, bits in {8, 4, 2} (K, V
// point to the packed codes).
hipError_t launch_decode_quant(int bits, int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s);

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

// Device address of the library's own split-decode workspace on the current
// device (H2O_SPLIT_SCRATCH_BYTES bytes), looked up once per device.
hipError_t split_scratch(void** ptr);

// Plain attention of one query over a contiguous cache of n_used rows.
hipError_t launch_fullcache(int dtype, int head_dim, int G, const DecodeArgs& a, hipStream_t s);

}  // namespace h2o
