// Device-side helpers shared by the HIP kernels: element types, 16-byte
// vector loads/stores and the FP8 E4M3 conversions of gfx950.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct fp8_t {
  uint8_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int bytes = 4;
};
template <>
struct Elem<half_t> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<fp8_t> {
  static constexpr int bytes = 1;
};

// 16 bytes held in four 32-bit registers.
struct alignas(16) Vec16 {
  uint32_t w[4];
};

__device__ __forceinline__ Vec16 load16(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return Vec16{{v.x, v.y, v.z, v.w}};
}

// K/V rows are read once per step: mark the loads non-temporal (streamed).
#ifndef PA_KV_NONTEMPORAL
#define PA_KV_NONTEMPORAL 1
#endif
__device__ __forceinline__ Vec16 load16_stream(const void* p) {
#if PA_KV_NONTEMPORAL
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return Vec16{{v[0], v[1], v[2], v[3]}};
#else
  return load16(p);
#endif
}

__device__ __forceinline__ void store16(void* p, const Vec16& v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(half2_t, w)[0]);
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(half2_t, w)[1]);
}

// OCP FP8 E4M3 -> two floats (bytes 0,1 of w when hi is false, else 2,3).
// The hardware conversion is exact.
__device__ __forceinline__ float2_t e4m3x2_to_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true)
            : __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}

// Saturate to the largest finite E4M3 magnitude, keeping NaN.
__device__ __forceinline__ float e4m3_clamp(float x) {
  return (x != x) ? x : __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
}

// Four floats -> four E4M3 bytes (little-endian order a, b, c, d), rounded to
// nearest even by the hardware conversion after saturation.  Every NaN is
// stored as 0x7F whatever its sign (a NaN's sign carries no meaning).
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), v, true);
  uint32_t r = static_cast<uint32_t>(v);
  r = (a != a) ? ((r & 0xFFFFFF00u) | 0x0000007Fu) : r;
  r = (b != b) ? ((r & 0xFFFF00FFu) | 0x00007F00u) : r;
  r = (c != c) ? ((r & 0xFF00FFFFu) | 0x007F0000u) : r;
  r = (d != d) ? ((r & 0x00FFFFFFu) | 0x7F000000u) : r;
  return r;
}

// Eight f16 numbers (one 16-byte chunk) -> eight E4M3 bytes of x * inv.
__device__ __forceinline__ uint2 f16x8_to_e4m3(const Vec16& v, float inv) {
  return make_uint2(f32x4_to_e4m3(half_lo(v.w[0]) * inv, half_hi(v.w[0]) * inv, half_lo(v.w[1]) * inv,
                                  half_hi(v.w[1]) * inv),
                    f32x4_to_e4m3(half_lo(v.w[2]) * inv, half_hi(v.w[2]) * inv, half_lo(v.w[3]) * inv,
                                  half_hi(v.w[3]) * inv));
}

// Four f32 numbers (one 16-byte chunk) -> four E4M3 bytes of x * inv.
__device__ __forceinline__ uint32_t f32x4_chunk_to_e4m3(const Vec16& v, float inv) {
  return f32x4_to_e4m3(__builtin_bit_cast(float, v.w[0]) * inv, __builtin_bit_cast(float, v.w[1]) * inv,
                       __builtin_bit_cast(float, v.w[2]) * inv, __builtin_bit_cast(float, v.w[3]) * inv);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(half_t x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ half_t from_f32<half_t>(float x) {
  return static_cast<half_t>(x);  // round to nearest even
}

}  // namespace pa
