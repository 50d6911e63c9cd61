// index_prep_dev.hpp -- per-row Hadamard + quantisation, shared by the
// standalone prep kernel and the indexer's fused query prologue.
#pragma once
#include "csa_device.hpp"
#include "../../include/csa.h"

namespace csa {

template <bool kF32In>
__device__ __forceinline__ void load_pair(const void* v, int64_t idx, float& x0, float& x1) {
  if (kF32In) {
    float2 t = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(v) + idx);
    x0 = t.x;
    x1 = t.y;
  } else {
    uint32_t t = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(v) + idx);
    x0 = __uint_as_float(t << 16);
    x1 = __uint_as_float(t & 0xFFFF0000u);
  }
}

// Rotary embedding of one row held two elements per lane (lane index li
// within the row holds elements 2 li, 2 li + 1, an adjacent pair): the pairs
// of the last rope_dim dims are rotated by the (cos, sin) of the row's
// position, in fp32 ("Token 的一生：DSV4 架构与 DSpark" §4: rope before the
// Hadamard rotation and the quantisation).
template <int D>
__device__ __forceinline__ void rope_pair(float& x0, float& x1, int li, int64_t pos,
                                          const float* __restrict__ cos_sin, int rope_dim) {
  const int i = li - (D - rope_dim) / 2;
  if (i >= 0) {
    const float2 cs = reinterpret_cast<const float2*>(cos_sin)[pos * (rope_dim / 2) + i];
    const float a = x0 * cs.x - x1 * cs.y;
    const float b = x0 * cs.y + x1 * cs.x;
    x0 = a;
    x1 = b;
  }
}

// Rotate (optionally) and quantise one row of D in {64, 128} held two elements
// per lane (D == 64: a half-wave per row), and store it as output row `dst`.
// Every lane of the wave must call this (it uses cross-lane shuffles).
//   FP8:   out uint8 [*][D], out_scale float [*]: scale = max(amax, FLT_MIN)/448,
//          code = e4m3(x / scale)
//   MXFP4: out uint8 [*][D/2] (element 2i in the low nibble), out_scale uint8
//          [*][D/32]: X = floor(log2 amax) - 2, code = e2m1(x * 2^-X), byte X+127
//   F32:   out float [*][D]
template <int D>
__device__ __forceinline__ void prep_and_store(float x0, float x1, bool valid, bool hadamard,
                                               int out_fmt, void* out, void* out_scale,
                                               int64_t dst) {
  const int lane = threadIdx.x & 63;
  const int li = (D == 64) ? (lane & 31) : lane;  // lane index within the row
  if (hadamard) {
    if (D == 128) fwht128_wave(x0, x1);
    else fwht64_halfwave(x0, x1);
  }
  if (out_fmt == CSA_FP8_E4M3) {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = group_max<D / 2>(amax);
    const float sc = fmaxf(amax, kFltMin) / kE4m3Max;
    const uint32_t c = e4m3x2(x0 / sc, x1 / sc);
    if (valid) {
      reinterpret_cast<uint16_t*>(out)[dst * (D / 2) + li] = (uint16_t)c;
      if (li == 0) reinterpret_cast<float*>(out_scale)[dst] = sc;
    }
  } else if (out_fmt == CSA_MXFP4) {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = group_max<16>(amax);  // 32 elements = 16 lanes
    const int X = mx_block_exponent(amax);
    const uint32_t c = f32_to_e2m1(ldexpf(x0, -X)) | (f32_to_e2m1(ldexpf(x1, -X)) << 4);
    if (valid) {
      reinterpret_cast<uint8_t*>(out)[dst * (D / 2) + li] = (uint8_t)c;
      if ((li & 15) == 0) reinterpret_cast<uint8_t*>(out_scale)[dst * (D / 32) + (li >> 4)] = (uint8_t)(X + 127);
    }
  } else {
    if (valid) *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + dst * D + 2 * li) = make_float2(x0, x1);
  }
}

}  // namespace csa
