// csa_device.hpp -- device helpers shared by the CSA / HCA kernels (gfx950).
//
// Number formats: OCP e4m3fn (FP8, max 448), OCP MX v1.0 MXFP4 (e2m1 + e8m0),
// bfloat16. Sources for where they are used: "Token 的一生：DSV4 架构与 DSpark"
// §3.1 / §4 (FP8 / FP4 indexer after a Hadamard rotation) and "DeepSeek-V4 的
// 交錯壓縮注意力（CSA/HCA）" section "低精度與儲存策略的配合" (FP8 KV, BF16 RoPE).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

constexpr int kWave = 64;
constexpr int kKvDim = 576;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kTopK = 512;
constexpr float kE4m3Max = 448.0f;
constexpr float kFltMin = 1.17549435e-38f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- FP8 e4m3fn
// Round-to-nearest-even, saturating at +-448, sign kept (also for zero).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fminf(fabsf(x), kE4m3Max);
  uint32_t ua = __float_as_uint(a);
  int e = (int)(ua >> 23) - 127;
  if (e < -6) {  // e4m3 subnormal range: value = m * 2^-9
    float m = rintf(a * 512.0f);  // exact scaling, RNE; m == 8 is the min normal
    return sign | (uint32_t)m;
  }
  uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);  // RNE to 3 mantissa bits
  uint32_t eb = (r >> 23) - 120u;                   // rebias 127 -> 7
  return sign | (eb << 3) | ((r >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -v : v;
}

// bf16 bits of an e4m3 code (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  return __float_as_uint(e4m3_to_f32(c)) >> 16;
}

// ---------------------------------------------------------------- MXFP4
// e2m1 code of x (already divided by the block scale), nearest even, saturating at 6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  float a = fabsf(x);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
  float v = mag[c & 7u];
  return (c & 8u) ? -v : v;
}

// Shared block exponent X = floor(log2 amax) - 2 (emax of e2m1), -127 for 0,
// clamped to the e8m0 range.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  int X = (ef == 0) ? -127 : (int)ef - 127 - 2;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Max over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Fast Walsh-Hadamard transform of a 128-vector held two elements per lane
// (lane l holds elements 2l and 2l+1), spans 1, 2, 4, ..., 64 in that order,
// fp32, then scaled by 1/sqrt(128): y = H_128 x / sqrt(128), Sylvester order
// ("Token 的一生：DSV4 架构与 DSpark" §4: rotate before FP8/FP4 quantisation).
__device__ __forceinline__ void fwht128_wave(float& x0, float& x1) {
  const int lane = threadIdx.x & 63;
  float a = x0, b = x1;
  x0 = a + b;
  x1 = a - b;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    float p0 = __shfl_xor(x0, m, kWave);
    float p1 = __shfl_xor(x1, m, kWave);
    bool upper = (lane & m) != 0;
    x0 = upper ? (p0 - x0) : (x0 + p0);
    x1 = upper ? (p1 - x1) : (x1 + p1);
  }
  const float s = 0.0883883476483184405f;  // 1/sqrt(128) rounded to fp32
  x0 *= s;
  x1 *= s;
}

// 64-element variant (lane l < 32 holds 2l, 2l+1; lanes 32..63 hold the
// second vector of a pair of rows processed together).
__device__ __forceinline__ void fwht64_halfwave(float& x0, float& x1) {
  const int lane = threadIdx.x & 31;
  float a = x0, b = x1;
  x0 = a + b;
  x1 = a - b;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    float p0 = __shfl_xor(x0, m, kWave);
    float p1 = __shfl_xor(x1, m, kWave);
    bool upper = (lane & m) != 0;
    x0 = upper ? (p0 - x0) : (x0 + p0);
    x1 = upper ? (p1 - x1) : (x1 + p1);
  }
  const float s = 0.125f;  // 1/sqrt(64)
  x0 *= s;
  x1 *= s;
}

// Order-preserving uint32 key of a float for "larger is better" selection:
// -0 maps to +0, NaN ranks below -inf (key 0).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace csa
