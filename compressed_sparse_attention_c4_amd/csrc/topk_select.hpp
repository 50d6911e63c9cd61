// topk_select.hpp -- the top-512 radix select of one workgroup, shared by the
// top-512 kernel and the indexer's fused candidate pass ("Token 的一生：DSV4
// 架构与 DSpark" §3.2: top-512 of the indexer logits).
//
// Order: larger key first, equal keys by lower element index. Keys are the
// order-preserving uint32 image of the logit; key 0 (NaN, or an absent
// element) ranks below every other key.
#pragma once
#include "csa_device.hpp"

namespace csa {

constexpr int kTopkBins = 3072;     // >= 2049 buckets, multiple of every workgroup size
constexpr int kTopkCandCap = 2048;  // threshold-bucket keys listed in LDS
constexpr int kTopkMaxWaves = 16;   // largest workgroup: 1024 threads

// LDS working set of one selection of at most kK elements.
template <int kK>
struct TopkLdsT {
  uint32_t hist[kTopkBins];
  uint32_t red[2 * kTopkMaxWaves];
  uint32_t sel_bin, sel_above;
  uint32_t list_n;                 // length of the threshold bucket's list
  uint32_t thr, need;              // threshold of a short bucket
  uint32_t cand[kTopkCandCap];     // keys of the threshold bucket
  int32_t out_e[kK];               // element placed at each output position
  uint32_t out_k[kK];              // and its key
};
using TopkLds = TopkLdsT<kTopK>;

// Exclusive scan of one uint32 per wave (value taken from lane 0 of each
// wave) over the workgroup's TH/64 waves; returns this wave's offset, sets total.
// kTail = false leaves out the closing barrier (which keeps sh from being
// overwritten while a wave still reads it) where a later barrier comes first.
template <int TH, bool kTail = true>
__device__ __forceinline__ uint32_t wave_offsets(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int w = 0; w < TH / 64; ++w) {
    const uint32_t x = sh[w];
    off += (w < wave) ? x : 0u;
    tot += x;
  }
  if (kTail) __syncthreads();
  total = tot;
  return off;
}

// hist[bin] += 1 for every lane with valid set. Lanes that hit the same bin
// are merged into one atomic while groups are large; once a peeled group is a
// single lane the rest add directly.
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t bin, bool valid) {
  const int lane = threadIdx.x & 63;
  uint64_t active = __ballot(valid);
  for (int it = 0; it < 8 && active; ++it) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(valid && bin == lb) & active;
    const uint32_t cnt = (uint32_t)__popcll(same);
    if (lane == leader) atomicAdd(&hist[lb], cnt);
    active &= ~same;
    if (cnt == 1) break;
  }
  if ((active >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

// Bucket (scanning from the top of hist[0..nbins)) where the running count
// reaches k; *sel_bin = bucket, *sel_above = count strictly above it.
template <int TH>
__device__ __forceinline__ void find_bucket(const uint32_t* hist, int nbins, uint32_t k,
                                            uint32_t* scan_sh, uint32_t* sel_bin,
                                            uint32_t* sel_above) {
  const int per = nbins / TH;
  uint32_t c = 0;
  for (int q = 0; q < per; ++q) c += hist[nbins - 1 - per * threadIdx.x - q];
  // block exclusive scan of c in thread order (thread 0 = top bins)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  (void)lane;
  (void)wave;
  const uint32_t x = wave_inclusive_scan(c);
  uint32_t tot;
  const uint32_t woff =
      wave_offsets<TH, false>((uint32_t)__builtin_amdgcn_readlane((int)x, 63), scan_sh, tot);
  uint32_t above = woff + x - c;
  if (above < k && above + c >= k) {
    for (int q = 0; q < per; ++q) {
      const int bin = nbins - 1 - per * threadIdx.x - q;
      const uint32_t h = hist[bin];
      if (above + h >= k) {
        *sel_bin = (uint32_t)bin;
        *sel_above = above;
        break;
      }
      above += h;
    }
  }
  __syncthreads();
}

// Selects the K largest (K <= the Lds capacity) of the n elements held in registers (element
// seg + 64 i + lane is key kr[i] of this lane; elements >= n hold key 0) and
// parks them in L.out_e / L.out_k by output position, in ascending element
// order. K <= n. Every thread of the TH-thread workgroup calls it; L.hist must
// have been cleared by the workgroup before the call (the first barrier
// inside orders the clear before any use). Ends with a barrier.
// With kPay, two 32-bit payloads of each element (pa[i], pb[i], e.g. its
// entry index and slot, loaded with the key) are parked beside it, at
// topk_pay_a(L)[pos] and topk_pay_b(L)[pos] (K <= 512), so an emission needs
// no second round of loads.
template <class Lds>
__device__ __forceinline__ int32_t* topk_pay_a(Lds& L) {
  return reinterpret_cast<int32_t*>(L.cand);
}
template <class Lds>
__device__ __forceinline__ int32_t* topk_pay_b(Lds& L) {
  return reinterpret_cast<int32_t*>(L.cand) + kTopK;
}

template <int kE, int TH, bool kPay, class Lds>
__device__ __forceinline__ void topk_select_impl(const uint32_t (&kr)[kE], const int32_t (&pa)[kE],
                                                 const int32_t (&pb)[kE], int n, int K, int seg,
                                                 Lds& L) {
  static_assert(2 * kTopK <= kTopkCandCap, "payloads live in the threshold list's space");
  constexpr int kBins = kTopkBins;
  constexpr int kCandCap = kTopkCandCap;
  constexpr int kWaves = kTopkMaxWaves;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t* const hist = L.hist;
  uint32_t* const red = L.red;
  uint32_t& sel_bin = L.sel_bin;
  uint32_t& sel_above = L.sel_above;
  uint32_t& s_thr = L.thr;
  uint32_t& s_need = L.need;
  uint32_t* const s_cand = L.cand;
  int32_t* const s_out_e = L.out_e;
  uint32_t* const s_out_k = L.out_k;
  if (threadIdx.x == 0) L.list_n = 0u;  // ordered before its use by the barriers below
  uint32_t thr = 0, need = 0;
  const bool take_all = n <= K;  // every element is selected
  if (!take_all) {
    // ---- 1. key range of the non-NaN keys: the minimum of key - 1 (key 0
    // wraps to the top) plus one; the maximum is unaffected by key 0
    uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < kE; ++i) {
      kmin1 = min(kmin1, kr[i] - 1u);
      kmax = max(kmax, kr[i]);
    }
    kmin1 = wave_umin(kmin1);
    kmax = wave_umax(kmax);
    if (lane == 0) {
      red[wave] = kmin1;
      red[kWaves + wave] = kmax;
    }
    __syncthreads();
    kmin1 = 0xFFFFFFFFu;
    kmax = 0u;
    for (int w = 0; w < TH / 64; ++w) {
      kmin1 = min(kmin1, red[w]);
      kmax = max(kmax, red[kWaves + w]);
    }
    uint32_t kmin = kmin1 + 1u;  // 0 when every key is NaN (then kmax = 0 too)
    const uint32_t range = kmax - kmin;
    const int sh = range == 0u ? 0 : max(0, (32 - __clz(range)) - 11);
    auto bin_of = [&](uint32_t k) -> uint32_t { return k == 0u ? 0u : 1u + ((k - kmin) >> sh); };

    // ---- 2. bucket of the K-th largest key
#pragma unroll
    for (int i = 0; i < kE; ++i) atomicAdd(&hist[bin_of(kr[i])], 1u);
    __syncthreads();
    find_bucket<TH>(hist, kBins, (uint32_t)K, red, &sel_bin, &sel_above);
    const uint32_t bstar = sel_bin;
    uint32_t k = (uint32_t)K - sel_above;

    // ---- 3. exact threshold inside the bucket (its keys share everything
    // above the low sh bits of key - kmin; bucket 0 holds only key 0, so it
    // needs no refinement). The bucket's members are gathered into a short
    // LDS list when they fit.
    const uint32_t nb = hist[bstar];
    const bool listed = bstar != 0u && nb <= (uint32_t)kCandCap;
    if (listed) {
      // list_n was zeroed before the first barrier
#pragma unroll
      for (int i = 0; i < kE; ++i)
        if (bin_of(kr[i]) == bstar) s_cand[atomicAdd(&L.list_n, 1u)] = kr[i];
      __syncthreads();
    }
    uint32_t low = 0;  // threshold's low bits, built from the top
    int width = bstar == 0u ? 0 : sh;
    if (listed && nb <= (uint32_t)TH) {
      // a short bucket: each listed key counts the keys above and equal to
      // it; the key whose range of ranks covers k is the threshold (every
      // thread holding that key writes the same values)
      if (threadIdx.x < nb) {
        const uint32_t c = s_cand[threadIdx.x];
        uint32_t gt = 0, eq = 0;
        int i = 0;
        for (; i + 4 <= (int)nb; i += 4) {
          const uint4 x = *reinterpret_cast<const uint4*>(&s_cand[i]);
          gt += (x.x > c) + (x.y > c) + (x.z > c) + (x.w > c);
          eq += (x.x == c) + (x.y == c) + (x.z == c) + (x.w == c);
        }
        for (; i < (int)nb; ++i) {
          const uint32_t x = s_cand[i];
          gt += x > c;
          eq += x == c;
        }
        if (gt < k && k <= gt + eq) {
          s_thr = c;
          s_need = k - gt;
        }
      }
      __syncthreads();
      thr = s_thr;
      need = s_need;
      width = -1;  // done
    }
    uint32_t got_mask = 0;  // bits of the low part fixed so far
    while (width > 0) {
      const int w = min(11, width);
      const int shift = width - w;
      const uint32_t dmask = (1u << w) - 1u;
      __syncthreads();
      for (int i = threadIdx.x; i < kBins; i += TH) hist[i] = 0u;
      __syncthreads();
      if (listed) {
        for (int i = threadIdx.x; i < (int)nb; i += TH) {
          const uint32_t lo = (s_cand[i] - kmin) & ((1u << sh) - 1u);  // sh <= 21
          if ((lo & got_mask) == low) atomicAdd(&hist[(lo >> shift) & dmask], 1u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kE; ++i) {
          const uint32_t kk = kr[i];
          const uint32_t lo = (kk - kmin) & ((1u << sh) - 1u);
          const bool in = kk != 0u && bin_of(kk) == bstar && (lo & got_mask) == low;
          wave_hist_add(hist, (lo >> shift) & dmask, in);
        }
      }
      __syncthreads();
      find_bucket<TH>(hist, kBins, k, red, &sel_bin, &sel_above);
      k -= sel_above;
      low |= sel_bin << shift;
      got_mask |= dmask << shift;
      width -= w;
    }
    if (width == 0) {
      thr = bstar == 0u ? 0u : kmin + ((bstar - 1u) << sh) + low;
      need = k;
    }
  }

  // ---- 4. ordered placement: pos = #(key > thr before) + min(#(key == thr before), need).
  // Taking every present element is thr = 0 (NaN) with need = the present
  // NaNs, which come before the absent elements. Positions are settled from
  // ballots over the registers; the selected elements are parked in LDS by
  // position and emitted afterwards, one output position per thread, so the
  // index and page-table reads of all 512 run in parallel.
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    gt_w += (uint32_t)__popcll(__ballot(kr[i] > thr));
    eq_w += (uint32_t)__popcll(__ballot(kr[i] == thr));
  }
  uint32_t tot;
  const uint32_t off = wave_offsets<TH, false>(gt_w | (eq_w << 16), red, tot);
  if (take_all) need = (uint32_t)n - (tot & 0xFFFFu);
  uint32_t g = off & 0xFFFFu, q = off >> 16;
  const uint64_t lt = (1ull << lane) - 1ull;
  // the lane index again, by a route the compiler cannot match to the one the
  // loads used, so it does not keep kE element indices live in between
  const int lane_b = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const bool isgt = kr[i] > thr;
    const bool iseq = kr[i] == thr;
    const uint64_t bg = __ballot(isgt), be = __ballot(iseq);
    const uint32_t gb = g + (uint32_t)__popcll(bg & lt);
    const uint32_t qb = q + (uint32_t)__popcll(be & lt);
    if (isgt || (iseq && qb < need)) {
      const uint32_t pos = gb + min(qb, need);
      s_out_e[pos] = seg + 64 * i + lane_b;
      s_out_k[pos] = kr[i];
      if constexpr (kPay) {  // the list's keys are dead here (barriers since their last read)
        topk_pay_a(L)[pos] = pa[i];
        topk_pay_b(L)[pos] = pb[i];
      }
    }
    g += (uint32_t)__popcll(bg);
    q += (uint32_t)__popcll(be);
  }
  __syncthreads();
}

template <int kE, int TH, class Lds>
__device__ __forceinline__ void topk_select(const uint32_t (&kr)[kE], int n, int K, int seg,
                                            Lds& L) {
  const int32_t(&none)[kE] = reinterpret_cast<const int32_t(&)[kE]>(kr);
  topk_select_impl<kE, TH, false>(kr, none, none, n, K, seg, L);
}

template <int kE, int TH, class Lds>
__device__ __forceinline__ void topk_select_pay(const uint32_t (&kr)[kE], const int32_t (&pa)[kE],
                                                const int32_t (&pb)[kE], int n, int K, int seg,
                                                Lds& L) {
  topk_select_impl<kE, TH, true>(kr, pa, pb, n, K, seg, L);
}

}  // namespace csa
