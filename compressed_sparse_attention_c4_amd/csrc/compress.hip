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
#include "compress_dev.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kWavesPerWG = 4;

template <bool kF32In, bool kF32Out>
__global__ void __launch_bounds__(kWavesPerWG * 64)
compress_kernel(const void* __restrict__ x, const int32_t* __restrict__ cu_rows,
                const int32_t* __restrict__ start_pos, int ratio,
                const float* __restrict__ gate_w, const float* __restrict__ gate_b,
                const int32_t* __restrict__ page_table, int pt_stride,
                void* __restrict__ out_latent, float* __restrict__ out_scale,
                void* __restrict__ out_rope, int page_size) {
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int row0 = cu_rows[b];
  const int nrows = cu_rows[b + 1] - row0;
  const int s0 = start_pos[b];
  const int first = (s0 + ratio - 1) / ratio;  // first complete aligned block
  const int last = (s0 + nrows) / ratio;       // one past the last complete block
  const int kb = first + blockIdx.x * kWavesPerWG + wave;
  if (kb >= last) return;
  const int64_t rbase = (int64_t)row0 + (int64_t)kb * ratio - s0;

  const int64_t slot = (int64_t)page_table[(int64_t)b * pt_stride + kb / page_size] * page_size +
                       kb % page_size;
  compress_entry<kF32In, kF32Out>(x, rbase, ratio, gate_w, gate_b, slot, out_latent, out_scale,
                                  out_rope);
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
