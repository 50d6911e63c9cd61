// decode_prep.hip -- the per-sequence cache writes and the query preparation
// of one CSA decode step, in a single launch.
//
// "Token 的一生：DSV4 架构与 DSpark" §1 (the new token updates the compressed cache,
// the raw window and the indexer's K cache before the indexer runs), §2.1
// (block k = raw positions [4k, 4k+3], emitted once 4k+3 exists), §3.1 and §4
// (index-K rows and indexer queries: rope -> hadamard -> FP8 or FP4 quant, the
// rope at the token's position). The four writes are independent per sequence; as separate
// launches each costs a launch and a memory round trip for a few KB of work.
//
// Workgroup b < B handles sequence b with three wavefronts:
//   wave 0: if the token completes a block, the block's compressed entry
//           (softmax-gated pooling, as c4_compress) into the compressed pool;
//   wave 1: the token itself into the raw window pool (as c4_compress with
//           ratio 1: the row, quantised);
//   wave 2: if a block is completed, its index-K row (rotated, quantised, as
//           csa_index_prep) into the index pool at the block's entry.
// Workgroups from B on prepare the query rows, one row per wave and pass.
#include <algorithm>

#include "compress_dev.hpp"
#include "csa_internal.hpp"
#include "index_prep_dev.hpp"

namespace csa {
namespace {

constexpr int kWaves = 4;

template <bool kF32In, bool kF32Out, int D>
__global__ void __launch_bounds__(kWaves * 64)
decode_prep_kernel(const void* __restrict__ x, const int32_t* __restrict__ pos, int B, int ratio,
                   const float* __restrict__ gate_w, const float* __restrict__ gate_b,
                   const int32_t* __restrict__ pt, int pt_stride, void* __restrict__ c_lat,
                   float* __restrict__ c_sc, void* __restrict__ c_rope, int c_ps,
                   const int32_t* __restrict__ rpt, int rpt_stride, void* __restrict__ r_lat,
                   float* __restrict__ r_sc, void* __restrict__ r_rope, int r_ps,
                   const void* __restrict__ k_rows, const void* __restrict__ q_rows, bool kq_f32,
                   int64_t q_count, int H_I, bool hadamard, bool rope, const float* __restrict__ cos_sin,
                   int rope_dim, int kq_fmt, void* __restrict__ k_data,
                   void* __restrict__ k_scale, void* __restrict__ q_out,
                   void* __restrict__ q_out_scale) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int sub = (D == 64) ? (lane >> 5) : 0;            // row of a pair (D == 64)
  const int e0 = 2 * ((D == 64) ? (lane & 31) : lane);    // first element of this lane
  if ((int)blockIdx.x < B) {
    const int b = blockIdx.x;
    const int p = pos[b];
    const bool done = p + 1 >= ratio && (p + 1) % ratio == 0;  // the token completes a block
    const int kb = (p + 1) / ratio - 1;
    if (wave == 0) {
      if (!done) return;
      const int64_t slot = (int64_t)pt[(int64_t)b * pt_stride + kb / c_ps] * c_ps + kb % c_ps;
      compress_entry<kF32In, kF32Out>(x, (int64_t)b * ratio, ratio, gate_w, gate_b, slot, c_lat,
                                      c_sc, c_rope);
    } else if (wave == 1) {
      const int64_t slot = (int64_t)rpt[(int64_t)b * rpt_stride + p / r_ps] * r_ps + p % r_ps;
      compress_entry<kF32In, kF32Out>(x, (int64_t)b * ratio + ratio - 1, 1, gate_w, gate_b, slot,
                                      r_lat, r_sc, r_rope);
    } else if (wave == 2) {
      if (!done || k_rows == nullptr) return;
      const int64_t slot = (int64_t)pt[(int64_t)b * pt_stride + kb / c_ps] * c_ps + kb % c_ps;
      const bool valid = sub == 0;
      float x0 = 0.f, x1 = 0.f;
      if (valid) {
        if (kq_f32) load_pair<true>(k_rows, (int64_t)b * D + e0, x0, x1);
        else load_pair<false>(k_rows, (int64_t)b * D + e0, x0, x1);
        if (rope) rope_pair<D>(x0, x1, e0 / 2, p, cos_sin, rope_dim);
      }
      prep_and_store<D>(x0, x1, valid, hadamard, kq_fmt, k_data, k_scale, slot);
    }
    return;
  }
  if (q_rows == nullptr) return;
  constexpr int kRowsPerWave = 128 / D;
  const int64_t nwaves = (int64_t)(gridDim.x - B) * kWaves;
  for (int64_t r0 = ((int64_t)(blockIdx.x - B) * kWaves + wave) * kRowsPerWave; r0 < q_count;
       r0 += nwaves * kRowsPerWave) {
    const int64_t r = r0 + sub;
    const bool valid = r < q_count;
    float x0 = 0.f, x1 = 0.f;
    if (valid) {
      if (kq_f32) load_pair<true>(q_rows, r * D + e0, x0, x1);
      else load_pair<false>(q_rows, r * D + e0, x0, x1);
      if (rope) rope_pair<D>(x0, x1, e0 / 2, pos[r / H_I], cos_sin, rope_dim);
    }
    prep_and_store<D>(x0, x1, valid, hadamard, kq_fmt, q_out, q_out_scale, valid ? r : 0);
  }
}

}  // namespace

hipError_t launch_decode_prep(const DecodePrepArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int64_t q_count = a.q_rows ? (int64_t)a.B * a.H_I : 0;
  const int64_t rows_per_wg = kWaves * (128 / a.kpool.dim);
  int64_t qwg = (q_count + rows_per_wg - 1) / rows_per_wg;
  if (qwg > 1024) qwg = 1024;
  const dim3 grid((unsigned)(a.B + qwg));
  const bool f32_in = a.x_fmt == CSA_F32;
  const bool f32_out = a.c4.fmt == CSA_F32;
  const bool kq_f32 = a.kq_fmt == CSA_F32;
#define CSA_DP(FI, FO, D)                                                                        \
  hipLaunchKernelGGL((decode_prep_kernel<FI, FO, D>), grid, dim3(kWaves * 64), 0, s, a.x, a.pos,  \
                     a.B, a.ratio, a.gate_w, a.gate_b, a.page_table, a.pt_stride, a.c4.latent,     \
                     a.c4.latent_scale, a.c4.rope, a.c4.page_size, a.raw_page_table,               \
                     a.raw_pt_stride, a.raw.latent, a.raw.latent_scale, a.raw.rope,                \
                     a.raw.page_size, a.k_rows, a.q_rows, kq_f32, q_count, std::max(a.H_I, 1),     \
                     (a.flags & CSA_PREP_HADAMARD) != 0, (a.flags & CSA_PREP_ROPE) != 0,           \
                     a.rope.cos_sin, a.rope.dim, (int)a.kpool.fmt, a.kpool.data,                   \
                     a.kpool.scale, a.q_out, a.q_out_scale)
#define CSA_DP_D(FI, FO) \
  if (a.kpool.dim == 128) CSA_DP(FI, FO, 128); else CSA_DP(FI, FO, 64)
  if (f32_in && f32_out) { CSA_DP_D(true, true); }
  else if (f32_in) { CSA_DP_D(true, false); }
  else if (f32_out) { CSA_DP_D(false, true); }
  else { CSA_DP_D(false, false); }
#undef CSA_DP_D
#undef CSA_DP
  return hipGetLastError();
}

}  // namespace csa
