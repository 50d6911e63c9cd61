// topk.hip -- the fixed top-512 transform with page translation
// ("Token 的一生：DSV4 架构与 DSpark" §3.2: top-512 of logits[bs, c4_seqlen]
// under c4_seq_lens, translated through page_table to [bs, 512] physical
// indices, with optional raw (logical) indices; k fixed at 512).
//
// Order: larger logit first, equal logits by lower index; -0 equals +0; NaN
// ranks below -inf. Keys are the order-preserving uint32 image of the float.
//
// A 1024-thread workgroup holds up to 32768 keys of a row in registers (up to
// 32 per lane; wave w owns a contiguous segment, lane-interleaved so every load
// is coalesced), so the row is read from memory once and every pass below is
// register and LDS work. Selection is a radix select, never a sort:
//   1. the key range [kmin, kmax] of the row is found; keys are binned by
//      (key - kmin) >> sh into at most 2048 buckets (monotone in the key), so
//      logits that crowd into a narrow range still spread over the buckets;
//   2. a histogram (LDS; a wavefront merges the increments of lanes that hit
//      the same bucket) gives the bucket b* of the 512th largest key;
//   3. the keys inside b* are refined over their low bits (at most two more
//      histogram passes over the registers) to the exact threshold key and
//      the number of keys equal to it that are taken;
//   4. one ordered pass places every selected entry at
//      #(key > thr before it) + min(#(key == thr before it), need), using
//      wavefront ballots and one workgroup scan, which yields ascending index
//      order directly; the entries are parked in LDS by position and written
//      out (index and page lookups included) one position per thread.
// Longer rows (and long rows in small batches, to spread the work over more
// CUs) run in two launches: chunks of the row are reduced to their own top-512
// (key, index) in index order, then the candidates of all chunks are reduced
// again. Any entry of the row's top-512 is in its chunk's top-512, so the
// result is exact.
#include <limits.h>
#include <stdlib.h>

#include <algorithm>

#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "topk_select.hpp"

namespace csa {
namespace {

constexpr int kThreads = 1024;             // workgroup of whole rows and of the final merge
constexpr int kMaxE = 32;                    // keys per lane (held in registers)
constexpr int kRegRow = kThreads * kMaxE;    // longest row selected in one launch
constexpr int kTopkMaxK = 2048;              // largest k of the generic top-k

// kCandMerge: a group of `chunk` consecutive candidates of a row (several
// chunks' top-512 lists) reduced to its own top-512 list, candidates in and
// out (key, index, slot), so that a row with many chunks reaches the final
// pass with few candidates. Groups are contiguous and the output keeps the
// input's order, so the final pass sees the candidates in index order.
enum Mode { kRowFinal = 0, kChunkCand = 1, kCandFinal = 2, kCandMerge = 3 };

// ksel (<= kK) entries are selected per row; candidate lists and output rows
// hold ksel entries each.
template <int kMode, int kE, int TH, int kK>
__global__ void __launch_bounds__(TH)
topk_kernel(const float* __restrict__ logits, int64_t ld, const uint32_t* __restrict__ ckeys,
            const int32_t* __restrict__ cjs, const int32_t* __restrict__ cphys, int ncand, int chunk,
            const int32_t* __restrict__ row_len, const int32_t* __restrict__ row_seq,
            const int32_t* __restrict__ pt, int pt_stride, int c4_page_size, int ksel,
            int32_t* __restrict__ phys_idx, int32_t* __restrict__ logical_idx,
            uint32_t* __restrict__ okeys, int32_t* __restrict__ ojs, int32_t* __restrict__ ophys) {
  static_assert(kE >= 1 && kE <= kMaxE, "keys per lane");
  __shared__ TopkLdsT<kK> L;

  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = (int)min((int64_t)row_len[r], ld > 0 ? ld : (int64_t)INT_MAX);  // row_len <= ld
  // the elements this workgroup selects from, their keys and indices
  int n, base = 0;
  if (kMode == kRowFinal) {
    n = rl;
  } else if (kMode == kChunkCand) {
    base = blockIdx.x * chunk;
    n = max(0, min(chunk, rl - base));
  } else if (kMode == kCandMerge) {
    base = blockIdx.x * chunk;
    n = min(chunk, ncand - base);
  } else {
    n = ncand;
  }
  const int K = min(ksel, kMode == kCandFinal ? rl : n);  // entries to select
  const int seg = wave * 64 * kE;                          // first element of this wave

  // the histogram is cleared while the keys are in flight
  for (int i = threadIdx.x; i < kTopkBins; i += TH) L.hist[i] = 0u;
  // Keys stay in registers: element seg + 64 i + lane is key kr[i] of this
  // lane (coalesced loads, all issued at once). An element's index is
  // base + e, or (candidates) re-read at emission, which touches only the
  // selected ones. Absent elements (e >= n) read element 0 of the row and
  // take key 0, the key of NaN: they sort below every present element
  // (present NaNs come first by index), and K <= n, so none is ever selected
  // and no pass needs a separate validity mask.
  const int nv = n - seg - lane;  // element i of this lane exists iff 64*i < nv
  // Candidates of a 512-selection with few keys per lane load their entry
  // index and slot with the key; the select parks the selected ones' beside
  // them, so the emission reads them from LDS.
  constexpr bool kPay = (kMode == kCandFinal || kMode == kCandMerge) && kE <= 8 && kK == kTopK;
  uint32_t kr[kE];
  int32_t ja[kE], pa[kE];
  {
    const float* lrow = logits + (int64_t)r * ld + base;
    const int64_t c0 = (int64_t)r * ncand + (kMode == kCandMerge ? base : 0);
#pragma unroll
    for (int i = 0; i < kE; ++i) {
      const bool ok = 64 * i < nv;
      const int e = ok ? seg + 64 * i + lane : 0;
      const uint32_t k = (kMode == kCandFinal || kMode == kCandMerge) ? ckeys[c0 + e] : float_key(lrow[e]);
      kr[i] = ok ? k : 0u;
      if constexpr (kPay) {
        ja[i] = ok ? cjs[c0 + e] : -1;
        pa[i] = ok && cphys ? cphys[c0 + e] : -1;
      }
    }
  }
  if constexpr (kPay) topk_select_pay<kE, TH>(kr, ja, pa, n, K, seg, L);
  else topk_select<kE, TH>(kr, n, K, seg, L);
  // ---- emission (positions K..ksel-1 are padding)
  for (int p = threadIdx.x; p < ksel; p += TH) {
    if (kMode == kChunkCand) {
      const int64_t o = ((int64_t)r * gridDim.x + blockIdx.x) * ksel + p;
      okeys[o] = p < K ? L.out_k[p] : 0u;
      ojs[o] = p < K ? base + L.out_e[p] : INT_MAX;
    } else if (kMode == kCandMerge) {
      const int64_t o = ((int64_t)r * gridDim.x + blockIdx.x) * ksel + p;
      uint32_t key = 0u;
      int32_t j = INT_MAX, ph = -1;
      if (p < K) {
        key = L.out_k[p];
        if constexpr (kPay) {
          j = topk_pay_a(L)[p];
          ph = topk_pay_b(L)[p];
        } else {
          const int64_t c = (int64_t)r * ncand + base + L.out_e[p];
          j = cjs[c];
          ph = cphys[c];
        }
      }
      okeys[o] = key;
      ojs[o] = j;
      ophys[o] = ph;
    } else {
      int32_t phys = -1, j = -1;
      if (p < K) {
        const int e = L.out_e[p];
        if constexpr (kPay) j = topk_pay_a(L)[p];
        else j = kMode == kCandFinal ? cjs[(int64_t)r * ncand + e] : e;
        if (kMode == kCandFinal && cphys)  // candidates that carry their slot
          phys = kPay ? topk_pay_b(L)[p] : cphys[(int64_t)r * ncand + e];
        else
          phys = (int32_t)((int64_t)pt[(int64_t)row_seq[r] * pt_stride + j / c4_page_size] *
                               c4_page_size +
                           j % c4_page_size);
      }
      phys_idx[(int64_t)r * ksel + p] = phys;
      if (logical_idx) logical_idx[(int64_t)r * ksel + p] = j;
    }
  }
}

// keys per lane for n elements over th threads: the next power of two >= n / th
int keys_per_lane(int64_t n, int th) {
  int e = 1;
  while ((int64_t)e * th < n) e *= 2;
  return e;
}

// Launch of topk_kernel<kMode, e, th, kK> selecting ksel entries: kK = 512
// for ksel <= 512 (any workgroup size), else kK = 2048 (1024 threads).
template <int kMode>
void launch_mode(int th, int e, dim3 grid, hipStream_t s, const float* logits, int64_t ld,
                 const uint32_t* ckeys, const int32_t* cjs, const int32_t* cphys, int ncand, int chunk,
                 const int32_t* row_len, const int32_t* row_seq, const int32_t* pt, int pt_stride,
                 int c4_page_size, int32_t* phys_idx, int32_t* logical_idx, uint32_t* okeys,
                 int32_t* ojs, int32_t* ophys = nullptr, int ksel = kTopK) {
  if (ksel > kTopK) {
#define CSA_TOPK_LAUNCH_W(E)                                                                     \
  hipLaunchKernelGGL((topk_kernel<kMode, E, kThreads, kTopkMaxK>), grid, dim3(kThreads), 0, s,   \
                     logits, ld, ckeys, cjs, cphys, ncand, chunk, row_len, row_seq, pt,          \
                     pt_stride, c4_page_size, ksel, phys_idx, logical_idx, okeys, ojs, ophys)
    switch (e) {
      case 1: CSA_TOPK_LAUNCH_W(1); break;
      case 2: CSA_TOPK_LAUNCH_W(2); break;
      case 4: CSA_TOPK_LAUNCH_W(4); break;
      case 8: CSA_TOPK_LAUNCH_W(8); break;
      case 16: CSA_TOPK_LAUNCH_W(16); break;
      default: CSA_TOPK_LAUNCH_W(32); break;
    }
#undef CSA_TOPK_LAUNCH_W
    return;
  }
#define CSA_TOPK_LAUNCH(E, TH)                                                             \
  hipLaunchKernelGGL((topk_kernel<kMode, E, TH, kTopK>), grid, dim3(TH), 0, s, logits, ld,   \
                     ckeys, cjs, cphys, ncand, chunk, row_len, row_seq, pt, pt_stride,        \
                     c4_page_size, ksel, phys_idx, logical_idx, okeys, ojs, ophys)
#define CSA_TOPK_E(TH)                       \
  switch (e) {                               \
    case 1: CSA_TOPK_LAUNCH(1, TH); break;   \
    case 2: CSA_TOPK_LAUNCH(2, TH); break;   \
    case 4: CSA_TOPK_LAUNCH(4, TH); break;   \
    case 8: CSA_TOPK_LAUNCH(8, TH); break;   \
    case 16: CSA_TOPK_LAUNCH(16, TH); break; \
    default: CSA_TOPK_LAUNCH(32, TH); break; \
  }
  if (th == 256) {
    CSA_TOPK_E(256)
  } else if (th == 512) {
    CSA_TOPK_E(512)
  } else {
    CSA_TOPK_E(1024)
  }
#undef CSA_TOPK_E
#undef CSA_TOPK_LAUNCH
}

// How one launch_topk call splits its rows. Every workgroup holds at most 32
// keys per lane (16 preferred: 32 costs spills at 1024 threads).
//  - Whole rows, one 1024-thread workgroup each, when a row fits 16 keys per
//    lane and either the rows alone fill the GPU (>= 128) or they are short.
//  - Otherwise chunks of a row are reduced to their top-k candidates and the
//    candidates of a row are reduced again. With >= 128 rows (k = 512) the rows
//    already fill the GPU: chunks of 256 x 16 keys go to 256-thread workgroups,
//    several of which share a CU, so one workgroup's barrier waits overlap
//    another's work. Where chunks of 1024 x 16 keys on 1024-thread
//    workgroups still make at most 512 workgroups, those are taken instead,
//    so that the final pass has fewer candidates (128 rows x 32768: 8 chunks,
//    11.8 + 8.5 us; 2 chunks, 11.8 + 5.8 us).
//    With fewer rows, ~128 workgroups of 1024 threads, each >= 4096 keys.
//  - At most kRegRow / k chunks per row, so a row's candidates fit one final
//    workgroup. Rows longer than that are not supported (topk_max_len).
//  - k > 512 runs on 1024-thread workgroups only.
struct TopkPlan {
  bool whole_rows;
  int chunks, chunk, chunk_th, final_th;
};

TopkPlan topk_plan(int64_t R, int64_t ld, int k) {
  TopkPlan p{false, 1, (int)ld, kThreads, kThreads};
  if (ld <= kRegRow / 2 && (R >= 128 || ld <= 8192)) {
    p.whole_rows = true;
    return p;
  }
  const bool wide = k > kTopK;
  int64_t c;
  if (R >= 128 && !wide) {
    // 16 keys per lane; 1024-thread chunks while they still make about one
    // round of workgroups
    c = R * ((ld + kThreads * 16 - 1) / (kThreads * 16)) <= 512 ? kThreads * 16 : 256 * 16;
  } else {
    const int64_t want = (128 + R - 1) / R;
    c = std::max<int64_t>((ld + want - 1) / want, std::max<int64_t>(4096, 2 * (int64_t)k));
    c = std::min<int64_t>(c, kRegRow / 2);
  }
  int64_t chunks = (ld + c - 1) / c;
  if (chunks * k > kRegRow) chunks = kRegRow / k;
  c = (ld + chunks - 1) / chunks;
  p.chunks = (int)((ld + c - 1) / c);
  p.chunk = (int)c;
  p.chunk_th = (R >= 128 && !wide && c <= 256 * kMaxE) ? 256 : kThreads;
  p.final_th = (R >= 128 && !wide && (int64_t)p.chunks * k <= 256 * kMaxE) ? 256 : kThreads;
  return p;
}

}  // namespace

size_t topk_ws_bytes(int64_t R, int64_t max_len, int k) {
  const TopkPlan p = topk_plan(R, max_len, k);
  if (p.whole_rows) return 0;
  return (size_t)R * p.chunks * k * (sizeof(uint32_t) + sizeof(int32_t));
}

int64_t topk_max_len(int k) { return (int64_t)(kRegRow / k) * kRegRow; }

hipError_t launch_topk_cand_merge(const uint32_t* ckeys, const int32_t* cjs, const int32_t* cphys,
                                  int ncand, int group, int R, const int32_t* row_len,
                                  uint32_t* okeys, int32_t* ojs, int32_t* ophys, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int groups = (ncand + group - 1) / group;
  const int th = (R >= 128 && group <= 256 * kMaxE) ? 256 : kThreads;
  launch_mode<kCandMerge>(th, keys_per_lane(group, th), dim3(groups, R), s, nullptr, 0, ckeys, cjs,
                          cphys, ncand, group, row_len, nullptr, nullptr, 1, 64, nullptr, nullptr,
                          okeys, ojs, ophys);
  return hipGetLastError();
}

hipError_t launch_topk_cand_final(const uint32_t* ckeys, const int32_t* cjs, const int32_t* cphys,
                                  int ncand, int R,
                                  const int32_t* row_len, const int32_t* row_seq,
                                  const int32_t* page_table, int pt_stride, int c4_page_size,
                                  int32_t* phys_idx, int32_t* logical_idx, hipStream_t s) {
  if (R == 0) return hipSuccess;
  // (few rows: 512 threads; measured against 1024 for 32 rows x 4096
  // candidates: 5.7 vs 6.0 us)
  const int th = (R >= 128 && ncand <= 256 * kMaxE) ? 256 : (ncand <= 512 * 8 ? 512 : kThreads);
  launch_mode<kCandFinal>(th, keys_per_lane(ncand, th), dim3(1, R), s, nullptr, 0, ckeys, cjs,
                          cphys, ncand, 0, row_len, row_seq, page_table, pt_stride, c4_page_size,
                          phys_idx, logical_idx, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t ld, int R, const int32_t* row_len,
                       const int32_t* row_seq, const int32_t* page_table, int pt_stride,
                       int c4_page_size, int k, int32_t* phys_idx, int32_t* logical_idx, void* ws,
                       hipStream_t s) {
  if (R == 0) return hipSuccess;
  const TopkPlan p = topk_plan(R, ld, k);
  if (p.whole_rows) {
    launch_mode<kRowFinal>(kThreads, keys_per_lane(ld, kThreads), dim3(1, R), s, logits, ld,
                           nullptr, nullptr, nullptr, 0, 0, row_len, row_seq, page_table, pt_stride,
                           c4_page_size, phys_idx, logical_idx, nullptr, nullptr, nullptr, k);
    return hipGetLastError();
  }
  const int ncand = p.chunks * k;
  uint32_t* ck = (uint32_t*)ws;
  int32_t* cj = (int32_t*)((uint8_t*)ws + (size_t)R * ncand * sizeof(uint32_t));
  launch_mode<kChunkCand>(p.chunk_th, keys_per_lane(p.chunk, p.chunk_th), dim3(p.chunks, R), s,
                          logits, ld, nullptr, nullptr, nullptr, 0, p.chunk, row_len, row_seq, page_table,
                          pt_stride, c4_page_size, nullptr, nullptr, ck, cj, nullptr, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_mode<kCandFinal>(p.final_th, keys_per_lane(ncand, p.final_th), dim3(1, R), s, nullptr,
                          0, ck, cj, nullptr, ncand, 0, row_len, row_seq, page_table, pt_stride,
                          c4_page_size, phys_idx, logical_idx, nullptr, nullptr, nullptr, k);
  return hipGetLastError();
}

}  // namespace csa
