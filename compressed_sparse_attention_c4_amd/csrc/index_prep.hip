// index_prep.hip -- Hadamard rotation and FP8 / MXFP4 quantisation of indexer
// rows ("Token 的一生：DSV4 架构与 DSpark" §3.1: FP8 or FP4 query plus scale
// factors; §4: q and index-K go rope -> hadamard -> quant; RoPE is upstream).
//
// A wavefront prepares one 128-dim row (two elements per lane) or two 64-dim
// rows (one per half-wave); the rotation is a shuffle-based fast Walsh-Hadamard
// transform in registers, so the row is read once and written once.
#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "index_prep_dev.hpp"

namespace csa {
namespace {

constexpr int kWavesPerWG = 4;

template <int D, bool kF32In>
__global__ void __launch_bounds__(kWavesPerWG * 64)
index_prep_kernel(const void* __restrict__ v, int64_t rows, uint32_t flags, int out_fmt,
                  void* __restrict__ out, void* __restrict__ out_scale,
                  const int32_t* __restrict__ dst_rows) {
  constexpr int kRowsPerWave = 128 / D;
  const int lane = threadIdx.x & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerWG + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerWG;
  const int sub = (D == 64) ? (lane >> 5) : 0;       // which row of the pair
  const int e0 = 2 * ((D == 64) ? (lane & 31) : lane);  // first element of this lane
  for (int64_t r0 = wave_id * kRowsPerWave; r0 < rows; r0 += nwaves * kRowsPerWave) {
    const int64_t r = r0 + sub;
    const bool valid = r < rows;
    float x0 = 0.f, x1 = 0.f;
    if (valid) load_pair<kF32In>(v, r * D + e0, x0, x1);
    const int64_t d = valid ? (dst_rows ? (int64_t)dst_rows[r] : r) : 0;
    const bool store = valid && d >= 0;  // a negative destination skips the row
    prep_and_store<D>(x0, x1, store, flags & CSA_PREP_HADAMARD, out_fmt, out, out_scale,
                      store ? d : 0);
  }
}

}  // namespace

hipError_t launch_index_prep(const void* v, int v_fmt, int64_t rows, int dim, uint32_t flags,
                             int out_fmt, void* out, void* out_scale, const int32_t* dst_rows,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t rows_per_wg = kWavesPerWG * (128 / dim);
  int64_t nblocks = (rows + rows_per_wg - 1) / rows_per_wg;
  if (nblocks > 65536) nblocks = 65536;
  dim3 grid((unsigned)nblocks), block(kWavesPerWG * 64);
  const bool f32 = v_fmt == CSA_F32;
  if (dim == 128) {
    if (f32) hipLaunchKernelGGL((index_prep_kernel<128, true>), grid, block, 0, s, v, rows, flags, out_fmt, out, out_scale, dst_rows);
    else hipLaunchKernelGGL((index_prep_kernel<128, false>), grid, block, 0, s, v, rows, flags, out_fmt, out, out_scale, dst_rows);
  } else {
    if (f32) hipLaunchKernelGGL((index_prep_kernel<64, true>), grid, block, 0, s, v, rows, flags, out_fmt, out, out_scale, dst_rows);
    else hipLaunchKernelGGL((index_prep_kernel<64, false>), grid, block, 0, s, v, rows, flags, out_fmt, out, out_scale, dst_rows);
  }
  return hipGetLastError();
}

}  // namespace csa
