// Device helpers shared by the POET-X HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

typedef uint16_t bf16;  // bfloat16 bit pattern

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA A/B operand
typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ float bf2f(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest, ties to even; NaN stays NaN.
// float -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32;
// NaN stays NaN)
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_hw_t __attribute__((ext_vector_type(2)));

// two floats -> two packed bf16 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const bf16x2_hw_t h = __builtin_convertvector((f32x2_hw_t){lo, hi}, bf16x2_hw_t);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

__device__ __forceinline__ bf16 f2bf(float f) {
  const __bf16 h = (__bf16)f;
  bf16 u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// storage-type adaptors: the math is always fp32
template <typename TS> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct St<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16* p, float v) { *p = f2bf(v); }
};

// packed strict-upper-triangle index of (i, j), i < j, in a b x b block
__device__ __forceinline__ int tri_index(int i, int j, int b) {
  return i * b - (i * (i + 1)) / 2 + (j - i - 1);
}

// Q[i][j] of the skew-symmetric block whose packed parameters start at th
__device__ __forceinline__ float skew_at(const float* th, int i, int j, int b) {
  if (i < j) return th[tri_index(i, j, b)];
  if (i > j) return -th[tri_index(j, i, b)];
  return 0.0f;
}

// (i, j), i < j, of packed index t: row i holds t in [S(i), S(i+1)) with
// S(i) = i*b - i*(i+1)/2
__device__ __forceinline__ void tri_rc(int t, int b, int& i, int& j) {
  const float c = 2.0f * b - 1.0f;
  int r = (int)floorf(0.5f * (c - sqrtf(fmaxf(c * c - 8.0f * (float)t, 0.0f))));
  r = max(0, min(r, b - 2));
  while (r > 0 && r * b - r * (r + 1) / 2 > t) --r;
  while (r < b - 2 && (r + 1) * b - (r + 1) * (r + 2) / 2 <= t) ++r;
  i = r;
  j = t - (r * b - r * (r + 1) / 2) + r + 1;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace poetx
