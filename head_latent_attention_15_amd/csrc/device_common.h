// Device-side helpers shared by the HIP kernels of libmla (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// bf16 is carried as its raw 16-bit pattern.
typedef uint16_t bf16raw;

__device__ __forceinline__ float bf16_to_f32(bf16raw b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet), infinities stay infinite.
__device__ __forceinline__ bf16raw f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) {
    return (u & 0x007fffffu) ? static_cast<bf16raw>((u >> 16) | 0x0040u)
                             : static_cast<bf16raw>(u >> 16);
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16raw>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16raw> {
  static __device__ __forceinline__ float load(const bf16raw* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16raw* p, float v) { *p = f32_to_bf16(v); }
};

template <typename T> __device__ __forceinline__ float ld(const T* p) { return Elem<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v) { Elem<T>::store(p, v); }

// Rotation of one RoPE pair (x0, x1) at position pos for pair index k of a d-wide vector:
// angle pos * base^(-2k/d), evaluated in fp64 so that long positions keep full precision.
// rope_angle and rope_rotate are its two halves, for callers that compute the angle ahead
// of the values (same operations, same results).
__device__ __forceinline__ void rope_angle(int64_t pos, int k, int d, float base, double* s,
                                           double* c) {
  const double theta = pow(static_cast<double>(base), -2.0 * static_cast<double>(k) / d);
  const double ang = static_cast<double>(pos) * theta;
  sincos(ang, s, c);
}
__device__ __forceinline__ void rope_rotate(float x0, float x1, double s, double c, float* y0,
                                            float* y1) {
  *y0 = static_cast<float>(static_cast<double>(x0) * c - static_cast<double>(x1) * s);
  *y1 = static_cast<float>(static_cast<double>(x0) * s + static_cast<double>(x1) * c);
}
__device__ __forceinline__ void rope_pair(float x0, float x1, int64_t pos, int k, int d,
                                          float base, float* y0, float* y1) {
  double s, c;
  rope_angle(pos, k, d, base, &s, &c);
  rope_rotate(x0, x1, s, c, y0, y1);
}

// a * b rounded to fp32 on its own: never contracted into a following add (FMA), so a
// value compared against a maximum and later subtracted from it is the same number.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace mla
