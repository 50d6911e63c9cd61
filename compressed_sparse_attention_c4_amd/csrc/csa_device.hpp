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

// e4m3fn codes of a and b (low byte a), by the conversion instruction: round
// to nearest even, the same codes as f32_to_e4m3 for every |x| <= 460 (checked
// value by value on gfx950, midpoints and subnormals included); a NaN input
// gives the NaN code instead of f32_to_e4m3's 448.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
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
// Cross-lane moves stay on the vector ALU: DPP within 16-lane rows and the
// permlane swaps across rows. (The generic shuffle goes through the LDS
// crossbar, ds_bpermute, and the wave waits for its round trip.) Layouts:
// permlane16_swap(v, v) gives {row 2k's value, row 2k+1's value} to both rows
// 2k and 2k+1 (a row is 16 lanes); permlane32_swap(v, v) gives {the value of
// lane l % 32, the value of lane l % 32 + 32}.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowShl = 0x100;     // + n: lane l reads l + n within its row
constexpr int kDppRowShr = 0x110;     // + n: lane l reads l - n within its row
constexpr int kDppRowMirror = 0x140;  // lane l reads 15 - l within its row
constexpr int kDppRowHalfMirror = 0x141;  // lane l reads 7 - l within its half row

// The swaps are written as instructions: the compiler's generic combine of
// the swap intrinsic treats its two results as the same value and folds one
// into the other. The nops cover the VALU-write-to-permlane hazard.
__device__ __forceinline__ float2 permlane16_pair(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float2 permlane32_pair(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}

// Swap of two registers across rows: permlane16 gives a = [a.r0, b.r0, a.r2,
// b.r2], b = [a.r1, b.r1, a.r3, b.r3] (rows of 16 lanes); permlane32 gives
// a = [a.lo, b.lo], b = [a.hi, b.hi] (halves of 32 lanes).
__device__ __forceinline__ void permlane16_swap2(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap2(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// Four values per lane, p[k] = a row's partial of column group k: returns, in
// every lane of row r, the sum of p[r] over the four rows (a reduce-scatter:
// three swaps instead of four full reductions).
__device__ __forceinline__ float rows4_reduce_scatter(float p0, float p1, float p2, float p3) {
  permlane16_swap2(p0, p1);
  permlane16_swap2(p2, p3);
  float qa = p0 + p1, qb = p2 + p3;
  permlane32_swap2(qa, qb);
  return qa + qb;
}

// The value held by lane (l ^ kM), kM in {1, 2, 4, 8} (within a row).
template <int kM>
__device__ __forceinline__ float lane_xor(float v) {
  const int lane = threadIdx.x & 63;
  if constexpr (kM == 1) {
    return dpp_mov<kDppQuadXor1>(v);
  } else if constexpr (kM == 2) {
    return dpp_mov<kDppQuadXor2>(v);
  } else {
    static_assert(kM == 4 || kM == 8, "lane_xor: 1, 2, 4 or 8");
    const float from_below = dpp_mov<kDppRowShr + kM>(v);
    const float from_above = dpp_mov<kDppRowShl + kM>(v);
    return (lane & kM) ? from_below : from_above;
  }
}

// Max / sum over the 16 lanes of each row, in every lane of the row (every
// lane gets the bitwise same value).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppRowMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowHalfMirror>(v);
  return v + dpp_mov<kDppRowMirror>(v);
}
// Sum / max over the four lanes l % 16 + {0, 16, 32, 48}, in each of them.
__device__ __forceinline__ float cross_row_sum(float v) {
  const float2 a = permlane16_pair(v);
  const float2 b = permlane32_pair(a.x + a.y);
  return b.x + b.y;
}
__device__ __forceinline__ float cross_row_max(float v) {
  const float2 a = permlane16_pair(v);
  const float2 b = permlane32_pair(fmaxf(a.x, a.y));
  return fmaxf(b.x, b.y);
}
__device__ __forceinline__ float wave_sum(float v) { return cross_row_sum(row16_sum(v)); }
__device__ __forceinline__ float wave_max(float v) { return cross_row_max(row16_max(v)); }
// Unsigned 32-bit wave reductions and an inclusive wave scan on the same
// VALU paths (the permlane swaps move bits, so floats carry the integers).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dpp_u32<kDppQuadXor1>(v));
  v = min(v, dpp_u32<kDppQuadXor2>(v));
  v = min(v, dpp_u32<kDppRowHalfMirror>(v));
  v = min(v, dpp_u32<kDppRowMirror>(v));
  const float2 a = permlane16_pair(__uint_as_float(v));
  v = min(__float_as_uint(a.x), __float_as_uint(a.y));
  const float2 b = permlane32_pair(__uint_as_float(v));
  return min(__float_as_uint(b.x), __float_as_uint(b.y));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  const float2 a = permlane16_pair(__uint_as_float(v));
  v = max(__float_as_uint(a.x), __float_as_uint(a.y));
  const float2 b = permlane32_pair(__uint_as_float(v));
  return max(__float_as_uint(b.x), __float_as_uint(b.y));
}
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row feeds the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 feeds rows 2 and 3
// Inclusive prefix sum over the 64 lanes (lane order); lanes with no source
// in a DPP step add the 0 of the update's old value.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_u32<kDppRowShr + 1>(x);
  x += dpp_u32<kDppRowShr + 2>(x);
  x += dpp_u32<kDppRowShr + 4>(x);
  x += dpp_u32<kDppRowShr + 8>(x);
  x += dpp_u32<kDppRowBcast15, 0xA>(x);
  x += dpp_u32<kDppRowBcast31, 0xC>(x);
  return x;
}

// Max over groups of `width` consecutive lanes (16, 32 or 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
  static_assert(width == 16 || width == 32 || width == 64, "group_max: 16, 32 or 64 lanes");
  v = row16_max(v);
  if constexpr (width == 32) {
    const float2 a = permlane16_pair(v);
    v = fmaxf(a.x, a.y);
  } else if constexpr (width == 64) {
    v = cross_row_max(v);
  }
  return v;
}

// One butterfly span m across lanes: of the pair (a in the lane with bit m
// clear, b in its partner), the lower lane keeps a + b and the upper a - b.
template <int kM>
__device__ __forceinline__ void fwht_stage(float& x0, float& x1, int lane) {
  const bool upper = (lane & kM) != 0;
  if constexpr (kM <= 8) {
    const float p0 = lane_xor<kM>(x0);
    const float p1 = lane_xor<kM>(x1);
    x0 = upper ? (p0 - x0) : (x0 + p0);
    x1 = upper ? (p1 - x1) : (x1 + p1);
  } else {
    // the swap hands both lanes of a pair (a, b) = (lower's, upper's) value
    const float2 a = kM == 16 ? permlane16_pair(x0) : permlane32_pair(x0);
    const float2 b = kM == 16 ? permlane16_pair(x1) : permlane32_pair(x1);
    x0 = upper ? (a.x - a.y) : (a.x + a.y);
    x1 = upper ? (b.x - b.y) : (b.x + b.y);
  }
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
  fwht_stage<1>(x0, x1, lane);
  fwht_stage<2>(x0, x1, lane);
  fwht_stage<4>(x0, x1, lane);
  fwht_stage<8>(x0, x1, lane);
  fwht_stage<16>(x0, x1, lane);
  fwht_stage<32>(x0, x1, lane);
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
  fwht_stage<1>(x0, x1, lane);
  fwht_stage<2>(x0, x1, lane);
  fwht_stage<4>(x0, x1, lane);
  fwht_stage<8>(x0, x1, lane);
  fwht_stage<16>(x0, x1, lane);
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
