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

}  // namespace

hipError_t launch_index_prep(const void* v, int v_fmt, int64_t rows, int dim, uint32_t flags,
                             int out_fmt, void* out, void* out_scale, const int32_t* dst_rows,
                             const csa_rope& rope, hipStream_t s) {
  if (rows == 0) return hipSuccess;
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
