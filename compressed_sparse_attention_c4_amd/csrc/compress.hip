// compress.hip -- C4 / HCA compressor: softmax-gated pooling of `ratio` raw KV
// rows into one compressed entry, quantised into a paged KV pool.
//
// "Token 的一生：DSV4 架构与 DSpark" §2.1: block k covers raw positions
// [4k, 4k+3] and is emitted once position 4k+3 exists. "DeepSeek-V4 的交錯壓縮注意力
// （CSA/HCA）" CSA paragraph: softmax-gated pooling with a learned positional
// bias; HCA paragraph: the same at about 128x. Storage: "低精度與儲存策略的配合"
// (FP8 latent dims, BF16 RoPE dims).
//
// One wavefront per output entry. Lane l holds latent dims 8l..8l+7 (one
// 16-byte bf16 load per row) and RoPE dim 512+l, so every row is read with
// coalesced loads and the FP8 store of the entry is one 8-byte store per lane.
// The softmax over the block's rows runs online (running max and sum), so the
// rows are read once even for ratio 128; they are loaded four at a time, all
// four loads in flight together.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kWavesPerWG = 4;

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

template <bool kF32In, bool kF32Out>
__global__ void __launch_bounds__(kWavesPerWG * 64)
compress_kernel(const void* __restrict__ x, const int32_t* __restrict__ cu_rows,
                const int32_t* __restrict__ start_pos, int ratio,
                const float* __restrict__ gate_w, const float* __restrict__ gate_b,
                const int32_t* __restrict__ page_table, int pt_stride,
                void* __restrict__ out_latent, float* __restrict__ out_scale,
                void* __restrict__ out_rope, int page_size) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = cu_rows[b];
  const int nrows = cu_rows[b + 1] - row0;
  const int s0 = start_pos[b];
  const int first = (s0 + ratio - 1) / ratio;  // first complete aligned block
  const int last = (s0 + nrows) / ratio;       // one past the last complete block
  const int kb = first + blockIdx.x * kWavesPerWG + wave;
  if (kb >= last) return;
  const int64_t rbase = (int64_t)row0 + (int64_t)kb * ratio - s0;

  // the entry's page is looked up now, beside the row loads, not after them
  const int64_t slot = (int64_t)page_table[(int64_t)b * pt_stride + kb / page_size] * page_size +
                       kb % page_size;
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
  constexpr int kRowBatch = 4;
  for (int r0 = 0; r0 < ratio; r0 += kRowBatch) {
    float v[kRowBatch][9];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) load_row<kF32In>(x, rbase + (r0 + u < ratio ? r0 + u : 0), v[u]);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      // rows past the block get gate -inf: weight 0, and the running max
      // (finite from the block's first row on) is unchanged
      const bool in = r0 + u < ratio;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 9; ++i) d = fmaf(w[i], v[u][i], d);
      const float g = in ? wave_sum(d) + gate_b[in ? r0 + u : 0] : -INFINITY;
      const float mn = fmaxf(m, g);
      const float corr = expf(m - mn);  // exp(-inf) = 0 on the first row
      const float p = expf(g - mn);
      l = l * corr + p;
#pragma unroll
      for (int i = 0; i < 9; ++i) acc[i] = fmaf(p, v[u][i], acc[i] * corr);
      m = mn;
    }
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
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(c[i] / sc) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(c[4 + i] / sc) << (8 * i);
    uint8_t* lat = reinterpret_cast<uint8_t*>(out_latent) + slot * kLatent + 8 * lane;
    *reinterpret_cast<uint2*>(lat) = make_uint2(lo, hi);
    reinterpret_cast<uint16_t*>(out_rope)[slot * kRope + lane] = f32_to_bf16(c[8]);
    if (lane == 0) out_scale[slot] = sc;
  }
}

}  // namespace

hipError_t launch_compress(const void* x, int x_fmt, const int32_t* cu_rows,
                           const int32_t* start_pos, int B, int max_rows, int ratio,
                           const float* gate_w, const float* gate_b,
                           const int32_t* page_table, int pt_stride, const csa_kv_pool& out,
                           hipStream_t s) {
  const int max_blocks = max_rows / ratio + 1;
  dim3 grid((max_blocks + kWavesPerWG - 1) / kWavesPerWG, B);
  dim3 block(kWavesPerWG * 64);
  const bool f32_in = x_fmt == CSA_F32;
  const bool f32_out = out.fmt == CSA_F32;
#define CSA_LAUNCH_COMPRESS(FI, FO)                                                       \
  hipLaunchKernelGGL((compress_kernel<FI, FO>), grid, block, 0, s, x, cu_rows, start_pos, \
                     ratio, gate_w, gate_b, page_table, pt_stride, out.latent,           \
                     out.latent_scale, out.rope, out.page_size)
  if (f32_in && f32_out) CSA_LAUNCH_COMPRESS(true, true);
  else if (f32_in) CSA_LAUNCH_COMPRESS(true, false);
  else if (f32_out) CSA_LAUNCH_COMPRESS(false, true);
  else CSA_LAUNCH_COMPRESS(false, false);
#undef CSA_LAUNCH_COMPRESS
  return hipGetLastError();
}

}  // namespace csa
