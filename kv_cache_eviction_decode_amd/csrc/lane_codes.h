// Packed 8-, 4- and 2-bit cache codes as one lane reads them: 16 channels
// per lane, loaded with non-temporal loads, converted to fp32, packed on
// insert. Used by the decode kernels over caches of codes.
#pragma once

#include "h2o_device.h"

namespace h2o {

// Rows of codes (or of value grids) from `base` on as a raw buffer resource
// holding `bytes` bytes (>= 0): a load at or past that count returns zeros,
// range-checked by the load itself, so rows past the occupied ones need no
// clamp. The base must be the same in every lane (scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int bytes) {
  constexpr int kWord3 = 0x00020000;  // gfx9-family raw buffer: 32-bit data format, no swizzle
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, kWord3);
}
constexpr int kLoadNT = 2;  // cache-policy bit of a non-temporal buffer load

// A value the compiler must treat as opaque: keeps a masked code word from
// being folded into one bit-field extract per code, so that each code is
// converted by a single v_cvt_f32_ubyteN of its byte.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
  __asm__("" : "+v"(x));
  return x;
}

// to_float gives each channel's code times a power of two, weight(i), which
// the caller folds into the query (divide) and into the output accumulators
// (divide once at the end); multiplying by a power of two commutes with fp32
// rounding, so the results are those of the plain codes.
template <int BITS> struct LaneCodes;
template <> struct LaneCodes<8> {
  using T = uint4;
  __device__ __forceinline__ static constexpr float inv_weight(int) { return 1.0f; }
  __device__ __forceinline__ static T load(const uint8_t* p) { return ldnt16(p); }
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadNT));
  }
  __device__ __forceinline__ static void store(uint8_t* p, T v) { *reinterpret_cast<uint4*>(p) = v; }
  __device__ __forceinline__ static void to_float(T w, float (&c)[16]) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b) c[4 * i + b] = float((v[i] >> (8 * b)) & 0xFFu);
  }
  __device__ __forceinline__ static T pack(const uint32_t (&c)[16]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = c[4 * i] | c[4 * i + 1] << 8 | c[4 * i + 2] << 16 | c[4 * i + 3] << 24;
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct LaneCodes<4> {
  using T = uint2;
  __device__ __forceinline__ static T load(const uint8_t* p) { return ldnt8(p); }
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadNT));
  }
  __device__ __forceinline__ static void store(uint8_t* p, T v) { *reinterpret_cast<uint2*>(p) = v; }
  // Word i holds channels 8i..8i+7; masking the low and the high nibbles
  // in place leaves the even channels one per byte and the odd ones one per
  // byte times 16 (weight 16).
  __device__ __forceinline__ static constexpr float inv_weight(int i) { return (i & 1) ? 0.0625f : 1.0f; }
  __device__ __forceinline__ static void to_float(T w, float (&c)[16]) {
    const uint32_t v[2] = {w.x, w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t lo = opaque_u32(v[i] & 0x0F0F0F0Fu), hi = opaque_u32(v[i] & 0xF0F0F0F0u);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[8 * i + 2 * b] = float((lo >> (8 * b)) & 0xFFu);
        c[8 * i + 2 * b + 1] = float((hi >> (8 * b)) & 0xFFu);
      }
    }
  }
  __device__ __forceinline__ static T pack(const uint32_t (&c)[16]) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i / 8] |= c[i] << (4 * (i % 8));
    return make_uint2(w[0], w[1]);
  }
};
template <> struct LaneCodes<2> {
  using T = uint32_t;
  __device__ __forceinline__ static T load(const uint8_t* p) { return ldnt4(p); }
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadNT);
  }
  __device__ __forceinline__ static void store(uint8_t* p, T v) { *reinterpret_cast<uint32_t*>(p) = v; }
  // Byte b holds channels 4b..4b+3; the j-th crumb of every byte is channel
  // 4b + j, masked in place: one per byte times 4^j (weight 4^(i mod 4)).
  __device__ __forceinline__ static constexpr float inv_weight(int i) {
    return (i & 3) == 0 ? 1.0f : (i & 3) == 1 ? 0.25f : (i & 3) == 2 ? 0.0625f : 0.015625f;
  }
  __device__ __forceinline__ static void to_float(T w, float (&c)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t part = opaque_u32(w & (0x03030303u << (2 * j)));
#pragma unroll
      for (int b = 0; b < 4; ++b) c[4 * b + j] = float((part >> (8 * b)) & 0xFFu);
    }
  }
  __device__ __forceinline__ static T pack(const uint32_t (&c)[16]) {
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) w |= c[i] << (2 * i);
    return w;
  }
};

}  // namespace h2o
