// Device-side helpers shared by the OLMo 3 attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace olmo3 {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxHalfDim = 128;  // d <= 256

// RoPE rates of one layer, fp64, passed by value in the kernel arguments.
struct RopeTable {
  double inv_freq[kMaxHalfDim];
  float mscale;  // multiplier of rotated q and k (YaRN temperature, else 1)
};

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// Round-to-nearest-even fp32 -> bf16 (gfx950 converts with RNE in hardware).
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }

template <typename T> struct Io;
template <> struct Io<bf16> {
  static constexpr int kVec = 8;  // elements per 16-byte access
  typedef bf16x8 vec;
  __device__ static inline void to_f32(const vec& v, float* f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
  }
  __device__ static inline vec from_f32(const float* f) {
    vec v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)f[i];
    return v;
  }
};
template <> struct Io<float> {
  static constexpr int kVec = 4;
  typedef f32x4 vec;
  __device__ static inline void to_f32(const vec& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
  __device__ static inline vec from_f32(const float* f) {
    vec v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f[i];
    return v;
  }
};

// OCP e4m3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, largest finite value 448), converted in hardware on gfx950.
// The hardware rounds to nearest even but turns values past the largest
// finite one into NaN, so inputs are clamped to +-448 first (saturation).
// A NaN is passed through unclamped (min/max would replace it by a bound),
// so it is stored as a NaN code.
constexpr float kE4m3Max = 448.f;

__device__ __forceinline__ float e4m3_saturate(float x) {
  const float c = fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
  return __builtin_isnan(x) ? x : c;
}

// Four fp32 values -> four e4m3 codes, first value in the low byte.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  a = e4m3_saturate(a);
  b = e4m3_saturate(b);
  c = e4m3_saturate(c);
  d = e4m3_saturate(d);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Four e4m3 codes (low byte first) -> four fp32 values.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Map the hardware workgroup id so that consecutive logical work items land
// on the same XCD (workgroups are dealt round-robin over the 8 XCDs), which
// keeps items that share K/V in one XCD's L2.  Identity when n % 8 != 0.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcd = 8;
  if (n % kXcd) return bid;
  return (bid % kXcd) * (n / kXcd) + bid / kXcd;
}

}  // namespace olmo3
