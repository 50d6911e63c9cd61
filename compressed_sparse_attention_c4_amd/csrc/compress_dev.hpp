// compress_dev.hpp -- one compressed KV entry per wavefront: softmax-gated
// pooling of `ratio` raw rows and the store into a KV pool slot; shared by the
// compressor kernel and the fused decode preparation.
#pragma once
#include "csa_device.hpp"

namespace csa {

template <bool kF32In>
__device__ __forceinline__ void load_row(const void* x, int64_t row, float (&v)[9]) {
  const int lane = threadIdx.x & 63;
  if (kF32In) {
    const float* p = reinterpret_cast<const float*>(x) + row * kKvDim;
    float4 a = *reinterpret_cast<const float4*>(p + 8 * lane);
    float4 b = *reinterpret_cast<const float4*>(p + 8 * lane + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    v[8] = p[kLatent + lane];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + row * kKvDim;
    uint4 a = *reinterpret_cast<const uint4*>(p + 8 * lane);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    v[8] = bf16_to_f32(p[kLatent + lane]);
  }
}

// The entry pooled from rows rbase .. rbase + ratio - 1 of x, stored at
// `slot` of the pool (FP8 latent + scale + bf16 RoPE, or fp32). Every lane of
// the wave calls this; the page lookup for `slot` is the caller's.
template <bool kF32In, bool kF32Out>
__device__ __forceinline__ void compress_entry(const void* __restrict__ x, int64_t rbase, int ratio,
                                               const float* __restrict__ gate_w,
                                               const float* __restrict__ gate_b, int64_t slot,
                                               void* __restrict__ out_latent,
                                               float* __restrict__ out_scale,
                                               void* __restrict__ out_rope) {
  const int lane = threadIdx.x & 63;
  float w[9];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = gate_w[8 * lane + i];
  w[8] = gate_w[kLatent + lane];

  float m = -INFINITY, l = 0.f;
  float acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = 0.f;

  // rows in batches of kRowBatch, all loads of a batch issued before any of
  // its rows is used (rows past the block repeat its first row, unused)
  constexpr int kRowBatch = 4;  // (the batch sum of p below is written for four)
  for (int r0 = 0; r0 < ratio; r0 += kRowBatch) {
    float v[kRowBatch][9];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) load_row<kF32In>(x, rbase + (r0 + u < ratio ? r0 + u : 0), v[u]);
    // the batch's gates (independent reductions), then one rescale of the
    // running sums to the batch's maximum; rows past the block get gate -inf:
    // weight 0 (the block's first row keeps the maximum finite)
    float g[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      const bool in = r0 + u < ratio;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 9; ++i) d = fmaf(w[i], v[u][i], d);
      g[u] = in ? wave_sum(d) + gate_b[in ? r0 + u : 0] : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) mn = fmaxf(mn, g[u]);
    const float corr = expf(m - mn);  // exp(-inf) = 0 on the first batch
    float p[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) p[u] = expf(g[u] - mn);
    l = l * corr + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      float a = acc[i] * corr;
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) a = fmaf(p[u], v[u][i], a);
      acc[i] = a;
    }
    m = mn;
  }
  const float inv = 1.0f / l;
  float c[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) c[i] = acc[i] * inv;

  if (kF32Out) {
    float* lat = reinterpret_cast<float*>(out_latent) + slot * kLatent + 8 * lane;
    *reinterpret_cast<float4*>(lat) = make_float4(c[0], c[1], c[2], c[3]);
    *reinterpret_cast<float4*>(lat + 4) = make_float4(c[4], c[5], c[6], c[7]);
    reinterpret_cast<float*>(out_rope)[slot * kRope + lane] = c[8];
  } else {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(c[i]));
    amax = wave_max(amax);
    const float sc = fmaxf(amax, kFltMin) / kE4m3Max;
    const uint32_t lo = e4m3x2(c[0] / sc, c[1] / sc) | (e4m3x2(c[2] / sc, c[3] / sc) << 16);
    const uint32_t hi = e4m3x2(c[4] / sc, c[5] / sc) | (e4m3x2(c[6] / sc, c[7] / sc) << 16);
    uint8_t* lat = reinterpret_cast<uint8_t*>(out_latent) + slot * kLatent + 8 * lane;
    *reinterpret_cast<uint2*>(lat) = make_uint2(lo, hi);
    reinterpret_cast<uint16_t*>(out_rope)[slot * kRope + lane] = f32_to_bf16(c[8]);
    if (lane == 0) out_scale[slot] = sc;
  }
}

}  // namespace csa
