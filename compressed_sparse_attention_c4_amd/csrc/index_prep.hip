// index_prep.hip -- rotary embedding, Hadamard rotation and FP8 / MXFP4
// quantisation of indexer rows ("Token 的一生：DSV4 架构与 DSpark" §3.1: FP8 or
// FP4 query plus scale factors, prepared with the rope table and positions;
// §4: q and index-K go rope -> hadamard -> quant).
//
// A wavefront prepares one 128-dim row (two elements per lane) or two 64-dim
// rows (one per half-wave). A lane's two elements are an adjacent pair, so the
// rotary embedding is a 2 x 2 rotation in the lane; the Hadamard rotation is a
// shuffle-based fast Walsh-Hadamard transform in registers, so the row is read
// once and written once.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "index_prep_dev.hpp"

namespace csa {
namespace {

constexpr int kWavesPerWG = 4;
// Row slots a wave loads before preparing them: 8 for many rows (a slot's
// load latency then overlaps the others'), 1 for fewer, where the grid needs
// the workgroups more than a wave needs the overlap.
constexpr int kBatchMany = 8;
constexpr int64_t kManyRows = 65536;

// A wave takes kBatch row slots (a slot: one 128-dim row, or two 64-dim
// rows) at a time and issues all their loads (and rope-table reads) before it
// rotates and stores any.
template <int D, bool kF32In, int kBatch>
__global__ void __launch_bounds__(kWavesPerWG * 64)
index_prep_kernel(const void* __restrict__ v, int64_t rows, uint32_t flags, int out_fmt,
                  void* __restrict__ out, void* __restrict__ out_scale,
                  const int32_t* __restrict__ dst_rows, csa_rope rope) {
  constexpr int kRowsPerWave = 128 / D;
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerWG;
  const int sub = (D == 64) ? (lane >> 5) : 0;       // which row of the pair
  const int e0 = 2 * ((D == 64) ? (lane & 31) : lane);  // first element of this lane
  const bool do_rope = (flags & CSA_PREP_ROPE) != 0;
  for (int64_t b0 = wave_id * kBatch * kRowsPerWave; b0 < rows; b0 += nwaves * kBatch * kRowsPerWave) {
    float x0[kBatch], x1[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t r = b0 + i * kRowsPerWave + sub;
      x0[i] = x1[i] = 0.f;
      if (r < rows) load_pair<kF32In>(v, r * D + e0, x0[i], x1[i]);
    }
    if (do_rope) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t r = b0 + i * kRowsPerWave + sub;
        if (r < rows)
          rope_pair<D>(x0[i], x1[i], e0 / 2, rope.pos[r / rope.rows_per_pos], rope.cos_sin, rope.dim);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t r = b0 + i * kRowsPerWave + sub;
      const bool valid = r < rows;
      const int64_t d = valid ? (dst_rows ? (int64_t)dst_rows[r] : r) : 0;
      const bool store = valid && d >= 0;  // a negative destination skips the row
      prep_and_store<D>(x0[i], x1[i], store, flags & CSA_PREP_HADAMARD, out_fmt, out, out_scale,
                        store ? d : 0);
    }
  }
}

// 128-dim rows with FP8 or MXFP4 output, 16 lanes per row: lane s of a row
// holds its elements 8s .. 8s + 7, and a wave prepares four rows at once (two
// groups of four per step, so that eight rows' loads are in flight). Three of
// the Hadamard transform's seven butterfly spans run inside the lane and four
// across the row's 16 lanes (DPP moves), in the same order as fwht128_wave
// (spans 1, 2, 4, ..., 64), so the rotated values are the same; the row's
// maximum is a 16-lane reduction. A lane issues one 16-byte load (bf16) and
// one 8-byte (FP8) or 4-byte (MXFP4) store per row.
constexpr int kSegRows = 4;  // rows per wave at a time
constexpr int kSegGroups = 2;  // groups of four rows per wave and step

// A DPP move whose every lane has a source (no old value to keep).
template <int kCtrl>
__device__ __forceinline__ float dpp_full(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

// The value of lane l ^ kM (kM in {1, 2, 4, 8}) within the 16-lane row.
template <int kM>
__device__ __forceinline__ float row_xor(float v) {
  if constexpr (kM == 1) return dpp_full<kDppQuadXor1>(v);
  else if constexpr (kM == 2) return dpp_full<kDppQuadXor2>(v);
  else if constexpr (kM == 4) return dpp_full<0x1B>(dpp_full<kDppRowHalfMirror>(v));  // (l^7)^3
  else return dpp_full<0x128>(v);  // row_ror:8
}

// a / b rounded to nearest, from y = 1/b rounded to nearest and one correction
// of q = a y by the exact remainder a - b q (Markstein's method, which gives
// the correctly rounded quotient; checked against the division instruction
// sequence on 1.3e8 pairs of this kernel's ranges); the sign is a's, so that
// -0 / b stays -0.
__device__ __forceinline__ float div_rcp(float a, float b, float y) {
  const float q = a * y;
  const float r = fmaf(-b, q, a);
  return __builtin_copysignf(fmaf(r, y, q), a);
}

template <int kM>
__device__ __forceinline__ void seg_stage(float (&x)[8], int seg) {
  // of the pair (a in the lane with bit kM clear, b in its partner) the lower
  // lane keeps a + b and the upper a - b: fma(-1, b, a) = a - b, one rounding
  const float sgn = (seg & kM) ? -1.f : 1.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = row_xor<kM>(x[j]);
    x[j] = fmaf(sgn, x[j], p);
  }
}

__device__ __forceinline__ void fwht128_seg(float (&x)[8], int seg) {
#pragma unroll
  for (int m = 1; m < 8; m <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (!(j & m)) {
        const float a = x[j], b = x[j + m];
        x[j] = a + b;
        x[j + m] = a - b;
      }
  seg_stage<1>(x, seg);
  seg_stage<2>(x, seg);
  seg_stage<4>(x, seg);
  seg_stage<8>(x, seg);
  const float s = 0.0883883476483184405f;  // 1/sqrt(128) rounded to fp32
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= s;
}

template <bool kF32In, bool kFp4Out>
__global__ void __launch_bounds__(kWavesPerWG * 64)
index_prep128_kernel(const void* __restrict__ v, int64_t rows, uint32_t flags,
                     void* __restrict__ out, void* __restrict__ out_scale,
                     const int32_t* __restrict__ dst_rows, csa_rope rope) {
  constexpr int D = 128;
  constexpr int kStep = kSegRows * kSegGroups;  // rows per wave and step
  const int lane = threadIdx.x & 63;
  const int seg = lane & 15;
  const int rw = lane >> 4;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerWG;
  const bool do_rope = (flags & CSA_PREP_ROPE) != 0;
  const bool had = (flags & CSA_PREP_HADAMARD) != 0;
  const int rpp = rope.rows_per_pos;
  for (int64_t b0 = wave_id * kStep; b0 < rows; b0 += nwaves * kStep) {
    float x[kSegGroups][8];
#pragma unroll
    for (int i = 0; i < kSegGroups; ++i) {
      const int64_t r = min(b0 + i * kSegRows + rw, rows - 1);  // clamped: loads stay unconditional
      if (kF32In) {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(v) + r * D + 8 * seg);
        const float4 a = p[0], b = p[1];
        x[i][0] = a.x; x[i][1] = a.y; x[i][2] = a.z; x[i][3] = a.w;
        x[i][4] = b.x; x[i][5] = b.y; x[i][6] = b.z; x[i][7] = b.w;
      } else {
        const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(v) + r * D + 8 * seg);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[i][2 * k] = __uint_as_float(w[k] << 16);
          x[i][2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      }
    }
    if (do_rope) {
      // position of row b0 + k: q0 + (rem0 + k) / rpp, the division done once
      const int64_t bu = __builtin_amdgcn_readfirstlane((int)(b0 >> 32)) * 4294967296LL +
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)b0);
      const int64_t q0 = bu / rpp;
      const int rem0 = (int)(bu - q0 * rpp);
#pragma unroll
      for (int i = 0; i < kSegGroups; ++i) {
        const int t = rem0 + i * kSegRows + rw;
        const int64_t q = q0 + (rpp >= kStep ? (t >= rpp ? 1 : 0) : t / rpp);
        const int64_t r = b0 + i * kSegRows + rw;
        const int64_t pos = rope.pos[r < rows ? q : 0];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          rope_pair<D>(x[i][2 * k], x[i][2 * k + 1], 4 * seg + k, pos, rope.cos_sin, rope.dim);
      }
    }
#pragma unroll
    for (int i = 0; i < kSegGroups; ++i) {
      const int64_t r = b0 + i * kSegRows + rw;
      const bool valid = r < rows;
      const int64_t d = valid ? (dst_rows ? (int64_t)dst_rows[r] : r) : 0;
      const bool store = valid && d >= 0;  // a negative destination skips the row
      if (had) fwht128_seg(x[i], seg);
      if (!kFp4Out) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[i][j]));
        am = row16_max(am);
        const float sc = fmaxf(am, kFltMin) / kE4m3Max;
        const float y = 1.0f / sc;
        float qv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[j] = div_rcp(x[i][j], sc, y);  // = x / sc
        const uint32_t c0 = e4m3x2(qv[0], qv[1]) | (e4m3x2(qv[2], qv[3]) << 16);
        const uint32_t c1 = e4m3x2(qv[4], qv[5]) | (e4m3x2(qv[6], qv[7]) << 16);
        if (store) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(out) + d * D + 8 * seg) = make_uint2(c0, c1);
          if (seg == 0) reinterpret_cast<float*>(out_scale)[d] = sc;
        }
      } else {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[i][j]));
        am = fmaxf(am, dpp_mov<kDppQuadXor1>(am));  // a 32-element block: four lanes
        am = fmaxf(am, dpp_mov<kDppQuadXor2>(am));
        const int X = mx_block_exponent(am);
        uint32_t c = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) c |= f32_to_e2m1(ldexpf(x[i][j], -X)) << (4 * j);
        if (store) {
          reinterpret_cast<uint32_t*>(out)[d * (D / 8) + seg] = c;
          if ((seg & 3) == 0) reinterpret_cast<uint8_t*>(out_scale)[d * (D / 32) + (seg >> 2)] = (uint8_t)(X + 127);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_index_prep(const void* v, int v_fmt, int64_t rows, int dim, uint32_t flags,
                             int out_fmt, void* out, void* out_scale, const int32_t* dst_rows,
                             const csa_rope& rope, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dim == 128 && (out_fmt == CSA_FP8_E4M3 || out_fmt == CSA_MXFP4)) {
    const int64_t rows_per_wg = kWavesPerWG * kSegRows * kSegGroups;
    int64_t nb = (rows + rows_per_wg - 1) / rows_per_wg;
    if (nb > 65536) nb = 65536;
    const bool f32 = v_fmt == CSA_F32, fp4 = out_fmt == CSA_MXFP4;
#define CSA_IP128(F32, FP4)                                                                      \
  hipLaunchKernelGGL((index_prep128_kernel<F32, FP4>), dim3((unsigned)nb), dim3(kWavesPerWG * 64), \
                     0, s, v, rows, flags, out, out_scale, dst_rows, rope)
    if (f32) { if (fp4) CSA_IP128(true, true); else CSA_IP128(true, false); }
    else { if (fp4) CSA_IP128(false, true); else CSA_IP128(false, false); }
#undef CSA_IP128
    return hipGetLastError();
  }
  const int batch = rows >= kManyRows ? kBatchMany : 1;
  const int64_t rows_per_wg = kWavesPerWG * batch * (128 / dim);
  int64_t nblocks = (rows + rows_per_wg - 1) / rows_per_wg;
  if (nblocks > 65536) nblocks = 65536;
  dim3 grid((unsigned)nblocks), block(kWavesPerWG * 64);
  const bool f32 = v_fmt == CSA_F32;
#define CSA_IP(D, F32, B)                                                                        \
  hipLaunchKernelGGL((index_prep_kernel<D, F32, B>), grid, block, 0, s, v, rows, flags, out_fmt, \
                     out, out_scale, dst_rows, rope)
#define CSA_IP_B(D, F32)                 \
  if (batch == 1) CSA_IP(D, F32, 1);     \
  else CSA_IP(D, F32, kBatchMany);
  if (dim == 128) {
    if (f32) { CSA_IP_B(128, true) } else { CSA_IP_B(128, false) }
  } else {
    if (f32) { CSA_IP_B(64, true) } else { CSA_IP_B(64, false) }
  }
#undef CSA_IP_B
#undef CSA_IP
  return hipGetLastError();
}

}  // namespace csa
