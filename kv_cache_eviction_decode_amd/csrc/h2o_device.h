// Device-side helpers shared by the H2O kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h2o {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };

constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Loads of data read once per launch (the cache rows a decode step streams),
// marked non-temporal. Measured on this part: the OPT-6.7B decode step (278
// MB of rows, 4 layer caches in rotation) runs 15% faster than with plain
// loads.
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p)));
}
__device__ __forceinline__ uint2 ldnt8(const void* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(static_cast<const u32x2_nt*>(p)));
}
__device__ __forceinline__ uint32_t ldnt4(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Dot product of two 16-byte chunks (8 x 16-bit or 4 x fp32), fp32 accumulate.
template <int DT> __device__ __forceinline__ float dot16(uint4 a, uint4 b);

template <> __device__ __forceinline__ float dot16<DT_BF16>(uint4 a, uint4 b) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), s, false);
  return s;
}
template <> __device__ __forceinline__ float dot16<DT_F16>(uint4 a, uint4 b) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.x), __builtin_bit_cast(f16x2, b.x), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.y), __builtin_bit_cast(f16x2, b.y), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.z), __builtin_bit_cast(f16x2, b.z), s, false);
  s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a.w), __builtin_bit_cast(f16x2, b.w), s, false);
  return s;
}
template <> __device__ __forceinline__ float dot16<DT_F32>(uint4 a, uint4 b) {
  float s = __uint_as_float(a.x) * __uint_as_float(b.x);
  s = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), s);
  s = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), s);
  s = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), s);
  return s;
}

// Unpack a 16-byte chunk into fp32 values (8 for 16-bit types, 4 for fp32).
template <int DT> struct Unpack;
template <> struct Unpack<DT_BF16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(uint4 v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Unpack<DT_F16> {
  static constexpr int n = 8;
  __device__ __forceinline__ static void run(uint4 v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x2 h = __builtin_bit_cast(f16x2, w[i]);
      o[2 * i] = (float)h[0];
      o[2 * i + 1] = (float)h[1];
    }
  }
};
template <> struct Unpack<DT_F32> {
  static constexpr int n = 4;
  __device__ __forceinline__ static void run(uint4 v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

// Rows of d elements streamed with 16-byte loads: a row is read by LPR = d*bytes/16
// consecutive lanes, so one wave-wide load covers RPU = 64/LPR consecutive rows.
template <int DT, int D, int WAVES>
struct Shape {
  static constexpr int E = Elem<DT>::bytes;
  static constexpr int ROW = D * E;      // bytes per cache row
  static constexpr int LPR = ROW / 16;   // lanes per row
  static constexpr int RPU = 64 / LPR;   // rows per wave-wide load
  static constexpr int EPL = 16 / E;     // elements per lane
  static constexpr int NP = WAVES * RPU;  // online-softmax partials per workgroup
  static_assert(LPR >= 4 && LPR <= 64, "row must span 4..64 lanes");
};

// DPP lane permutations inside a 16-lane row.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

// Sum over aligned groups of N consecutive lanes (N in {4,8,16,32,64}); every
// lane of a group ends with the same (bitwise identical) value.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Wave issue priority (s_setprio takes an immediate, hence the switch).
__device__ __forceinline__ void set_wave_priority(int p) {
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// ---- cross-row exchanges without LDS (gfx950) --------------------------------
// v_permlane16_swap / v_permlane32_swap exchange rows of 16 lanes (odd rows
// with even rows) and the two 32-lane halves. Called with the same value as
// both operands they return, in every lane, the pair {even-side, odd-side}
// value in a fixed order, so a commutative combine of the pair is bitwise
// identical in both partner lanes.
struct LanePair {
  uint32_t lo, hi;
};
__device__ __forceinline__ LanePair swap16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}
constexpr int kRowRor8 = 0x128;  // lane i <- lane (i + 8) mod 16 within each row

// Combine values across the lane groups of N consecutive lanes (N in
// {4, 8, 16, 32}): lanes at the same position in every group end with the same
// result. OP is a commutative binary functor on floats.
template <int N, class OP> __device__ __forceinline__ float across_groups(float x, OP op) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N <= 4) x = op(x, __shfl_xor(x, 4));
  if constexpr (N <= 8) x = op(x, dpp<kRowRor8>(x));
  if constexpr (N <= 16) {
    const LanePair r = swap16(__float_as_uint(x));
    x = op(__uint_as_float(r.lo), __uint_as_float(r.hi));
  }
  if constexpr (N <= 32) {
    const LanePair r = swap32(__float_as_uint(x));
    x = op(__uint_as_float(r.lo), __uint_as_float(r.hi));
  }
  return x;
}
struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
  __device__ __forceinline__ float operator()(float a, float b) const { return fminf(a, b); }
};

// Combine within aligned groups of N consecutive lanes (N a power of two <= 64).
template <int N, class OP> __device__ __forceinline__ float lane_group(float x, OP op) {
#pragma unroll
  for (int off = 1; off < N; off <<= 1) x = op(x, __shfl_xor(x, off));
  return x;
}

// ---- cache codes (format: h2o_quant in the C header) ----------------------------
// BITS-wide codes, L = 2^BITS - 1. Grid step over [lo, hi] and the code of x:
// rint((x - mn) / scale) clamped to [0, L], ties to even, 0 on a degenerate
// grid. Plain fp32 operations with IEEE rounding (the divisions are correctly
// rounded), so the codes are exact.
template <int BITS> __device__ __forceinline__ float grid_scale(float lo, float hi) {
  return (hi - lo) / float((1 << BITS) - 1);
}
template <int BITS> __device__ __forceinline__ uint32_t quantize_code(float x, float scale, float mn) {
  if (!(scale > 0.f)) return 0;
  const float q = __builtin_rintf((x - mn) / scale);
  return uint32_t(fminf(fmaxf(q, 0.f), float((1 << BITS) - 1)));
}

// 16 consecutive channels of a code row held by one lane: 2 * BITS bytes,
// channel i at bit offset BITS * i of the lane's little-endian bytes. Loads
// are non-temporal (rows are streamed once per step).
template <int CTRL> __device__ __forceinline__ uint64_t dpp64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(x)), CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(x >> 32)), CTRL, 0xF, 0xF, false);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t min64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Minimum of a 64-bit key over the whole wave, in every lane (no LDS).
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t k) {
  k = min64(k, dpp64<kQuadSwap1>(k));
  k = min64(k, dpp64<kQuadSwap2>(k));
  k = min64(k, dpp64<kRowHalfMirror>(k));
  k = min64(k, dpp64<kRowMirror>(k));
  {
    const LanePair lo = swap16(uint32_t(k)), hi = swap16(uint32_t(k >> 32));
    k = min64((uint64_t(hi.lo) << 32) | lo.lo, (uint64_t(hi.hi) << 32) | lo.hi);
  }
  {
    const LanePair lo = swap32(uint32_t(k)), hi = swap32(uint32_t(k >> 32));
    k = min64((uint64_t(hi.lo) << 32) | lo.lo, (uint64_t(hi.hi) << 32) | lo.hi);
  }
  return k;
}

// Order-preserving key of a non-negative float and a position: the smallest
// key is the smallest score, and among equal scores the smallest position.
__device__ __forceinline__ uint64_t score_pos_key(float score, int32_t pos) {
  return (uint64_t(__float_as_uint(score)) << 32) | uint32_t(pos);
}

enum : int { POLICY_ACCUMULATED = 0, POLICY_AVERAGED = 1, POLICY_POSITION = 2 };

// Eviction key of a candidate at step t (the smallest leaves): its retention
// value under the policy, then its position. Accumulated: the score; averaged:
// the score over the t - pos + 1 queries that attended to it; position: the
// newest token leaves first.
__device__ __forceinline__ uint64_t evict_key(float score, int32_t pos, int32_t t, int policy) {
  if (policy == POLICY_POSITION) return uint64_t(uint32_t(0x7FFFFFFF - pos));
  const float v = policy == POLICY_AVERAGED ? score / float(t - pos + 1) : score;
  return score_pos_key(v, pos);
}

}  // namespace h2o
