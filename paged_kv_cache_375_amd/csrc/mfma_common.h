// Pieces of the decode kernels that run on the matrix cores (the grouped
// kernel and its prefix pass): the f16 MFMA, the transposing LDS read, exp2,
// the cross-row max, the exact E4M3 -> f16 conversion, and the swizzled LDS
// row layout of K and V chunks.
#pragma once
#include <hip/hip_runtime.h>

#include "device.h"

namespace pa {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int kChunk = 32;  // tokens per chunk: two 16-row tiles of the first product
constexpr float kLazy = 8.f;  // running-max slack, log2 units (weights <= 256)

__device__ __forceinline__ float4_t mfma16x16x32(const half8_t& a, const half8_t& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8_t as_half8(const Vec16& v) { return __builtin_bit_cast(half8_t, v); }

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// Transposing LDS read of 8 bytes per lane (see the header comment).
__device__ __forceinline__ short4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(const_cast<void*>(p)));
}

// exp2 on the hardware unit (inputs here are <= 0 or -inf; results below the
// smallest normal float may flush to zero, which no weight here relies on)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight E4M3 numbers (two 32-bit words) -> eight f16 (exact: every E4M3
// value is an f16 value).
__device__ __forceinline__ half8_t e4m3x8_to_half8(uint32_t lo, uint32_t hi) {
  half8_t r;
  const uint32_t w[2] = {lo, hi};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float2_t a = e4m3x2_to_f32(w[i], false), b = e4m3x2_to_f32(w[i], true);
    r[4 * i] = static_cast<_Float16>(a[0]);
    r[4 * i + 1] = static_cast<_Float16>(a[1]);
    r[4 * i + 2] = static_cast<_Float16>(b[0]);
    r[4 * i + 3] = static_cast<_Float16>(b[1]);
  }
  return r;
}

// Max over the four 16-lane rows of a wave, per lane column (lanes n, n + 16,
// n + 32, n + 48): gfx950's row swaps on the VALU, no LDS round trip.  (Each
// half of the swap result is copied to a scalar first: a bit-cast of one
// element of a vector result is lowered as element 0 by this compiler.)
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

// Sum over the four 16-lane rows, per lane column, the same way.
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

template <typename KV, int D>
struct Layout {
  static constexpr int KVB = Elem<KV>::bytes;
  static constexpr int NS = D / 32;             // k-steps of the first product
  static constexpr int NDT = D / 16;            // 16-wide head_dim tiles of the second
  static constexpr int VCH = D * KVB / 16;      // 16-byte pool chunks per token row
  static constexpr int NV = kChunk * VCH / 64;  // loads per lane per chunk, each of K and V
  static constexpr int LCH = D / 8;             // 16-byte f16 chunks per LDS row
  static_assert(NV >= 1 && (kChunk * VCH) % 64 == 0, "head_dim does not fit the load layout");
  // XOR swizzles of the 16-byte chunks of LDS row r.  K rows are read as
  // operand rows (16 consecutive rows, one chunk each): the row's low bits.
  // V rows are read by transposing reads (eight rows, a 32-byte column pair
  // each): twice the row's low bits.  Both keep the reads off shared banks.
  static __device__ __forceinline__ int swz_k(int r) { return r & (LCH - 1); }
  static __device__ __forceinline__ int swz_v(int r) { return (2 * r) & (LCH - 2); }
};

}  // namespace
}  // namespace pa
