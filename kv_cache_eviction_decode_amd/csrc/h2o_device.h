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

// Order-preserving key of a non-negative float and a position: the smallest
// key is the smallest score, and among equal scores the smallest position.
__device__ __forceinline__ uint64_t score_pos_key(float score, int32_t pos) {
  return (uint64_t(__float_as_uint(score)) << 32) | uint32_t(pos);
}

}  // namespace h2o
