// topk.hip -- the fixed top-512 transform with page translation
// ("Token 的一生：DSV4 架构与 DSpark" §3.2: top-512 of logits[bs, c4_seqlen]
// under c4_seq_lens, translated through page_table to [bs, 512] physical
// indices, with optional raw (logical) indices; k fixed at 512).
//
// Selection is a radix select on order-preserving 32-bit keys (no sort): three
// histogram passes over the row (11, 11 and 10 bits) find the exact key of the
// 512th largest entry and how many entries equal to it are taken (the lowest
// indices, which is the tie rule); one ordered compaction pass then writes the
// selected indices in ascending order. One 1024-thread workgroup per row; the
// histogram lives in LDS.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / 64;

// Exclusive scan of one uint32 per thread over the workgroup.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t s = lane < kWavesPerBlock ? sh[lane] : 0u;
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < kWavesPerBlock; o <<= 1) {
      uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane < kWavesPerBlock) sh[lane] = incl - s;
    if (lane == kWavesPerBlock - 1) sh[kWavesPerBlock] = incl;
  }
  __syncthreads();
  const uint32_t r = sh[wave] + x - v;
  total = sh[kWavesPerBlock];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kThreads)
topk512_kernel(const float* __restrict__ logits, int64_t ld, const int32_t* __restrict__ row_len,
               const int32_t* __restrict__ row_seq, const int32_t* __restrict__ pt, int pt_stride,
               int c4_page_size, int32_t* __restrict__ phys_idx, int32_t* __restrict__ logical_idx) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan_sh[kWavesPerBlock + 1];
  __shared__ uint32_t sel_digit, sel_above;

  const int r = blockIdx.x;
  const int n = row_len[r];
  const float* row = logits + (int64_t)r * ld;
  const int32_t* ptrow = pt + (int64_t)row_seq[r] * pt_stride;
  int32_t* out_p = phys_idx + (int64_t)r * kTopK;
  int32_t* out_l = logical_idx ? logical_idx + (int64_t)r * kTopK : nullptr;

  uint32_t thr = 0;   // key of the 512th largest (valid when n > 512)
  uint32_t need = 0;  // entries equal to thr that are taken
  if (n > kTopK) {
    uint32_t prefix = 0, pmask = 0, k = kTopK;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = shifts[pass];
      const int nbins = 1 << widths[pass];
      const uint32_t dmask = (uint32_t)nbins - 1u;
      for (int i = threadIdx.x; i < nbins; i += kThreads) hist[i] = 0;
      __syncthreads();
      for (int j = threadIdx.x; j < n; j += kThreads) {
        const uint32_t key = float_key(row[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      // Bins from the top: thread i takes bins nbins-1-per*i-q, q < per.
      const int per = nbins / kThreads;
      uint32_t c = 0;
      for (int q = 0; q < per; ++q) c += hist[nbins - 1 - per * threadIdx.x - q];
      uint32_t tot;
      uint32_t above = block_excl_scan(c, scan_sh, tot);
      if (above < k && above + c >= k) {
        for (int q = 0; q < per; ++q) {
          const int bin = nbins - 1 - per * threadIdx.x - q;
          const uint32_t h = hist[bin];
          if (above + h >= k) {
            sel_digit = (uint32_t)bin;
            sel_above = above;
            break;
          }
          above += h;
        }
      }
      __syncthreads();
      k -= sel_above;
      prefix |= sel_digit << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    thr = prefix;
    need = k;
  }

  // Ordered compaction: position of a selected j = #(key > thr before j)
  // + min(#(key == thr before j), need).
  uint32_t gt_before = 0, eq_before = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int j = base + threadIdx.x;
    uint32_t gt = 0, eq = 0;
    if (j < n) {
      if (n <= kTopK) {
        gt = 1;
      } else {
        const uint32_t key = float_key(row[j]);
        gt = key > thr;
        eq = key == thr;
      }
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan(gt | (eq << 16), scan_sh, tot);
    const uint32_t g = gt_before + (ex & 0xFFFFu);
    const uint32_t e = eq_before + (ex >> 16);
    if (gt || (eq && e < need)) {
      const uint32_t pos = g + min(e, need);
      const int64_t phys = (int64_t)ptrow[j / c4_page_size] * c4_page_size + j % c4_page_size;
      out_p[pos] = (int32_t)phys;
      if (out_l) out_l[pos] = j;
    }
    gt_before += tot & 0xFFFFu;
    eq_before += tot >> 16;
    if (gt_before + min(eq_before, need) >= (uint32_t)kTopK) break;
  }
  const int count = min(n, kTopK);
  for (int i = count + threadIdx.x; i < kTopK; i += kThreads) {
    out_p[i] = -1;
    if (out_l) out_l[i] = -1;
  }
}

}  // namespace

size_t topk_ws_bytes(int64_t, int64_t) { return 0; }

hipError_t launch_topk(const float* logits, int64_t ld, int R, const int32_t* row_len,
                       const int32_t* row_seq, const int32_t* page_table, int pt_stride,
                       int c4_page_size, int max_row_len, int32_t* phys_idx,
                       int32_t* logical_idx, void* ws, hipStream_t s) {
  (void)ws;
  (void)max_row_len;
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(topk512_kernel, dim3(R), dim3(kThreads), 0, s, logits, ld, row_len,
                     row_seq, page_table, pt_stride, c4_page_size, phys_idx, logical_idx);
  return hipGetLastError();
}

}  // namespace csa
