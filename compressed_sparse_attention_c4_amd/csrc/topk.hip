// topk.hip -- the fixed top-512 transform with page translation
// ("Token 的一生：DSV4 架构与 DSpark" §3.2: top-512 of logits[bs, c4_seqlen]
// under c4_seq_lens, translated through page_table to [bs, 512] physical
// indices, with optional raw (logical) indices; k fixed at 512).
//
// Order: larger logit first, equal logits by lower index; -0 equals +0; NaN
// ranks below -inf. Keys are the order-preserving uint32 image of the float.
//
// A 1024-thread workgroup holds up to 32768 keys of a row in LDS (wave w owns a
// contiguous segment, lane-interleaved so every load is coalesced), so the row
// is read from memory once. Selection is a radix select, never a sort:
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
//      order directly.
// Longer rows (and long rows in small batches, to spread the work over more
// CUs) run in two launches: chunks of the row are reduced to their own top-512
// (key, index) in index order, then the candidates of all chunks are reduced
// again. Any entry of the row's top-512 is in its chunk's top-512, so the
// result is exact.
#include <limits.h>

#include <algorithm>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 32;                    // keys per lane (held in LDS)
constexpr int kRegRow = kThreads * kMaxE;    // longest row selected in one launch
constexpr int kBins = 3072;                  // >= 2049 buckets, multiple of kThreads
constexpr int kCandCap = 2048;               // threshold-bucket keys listed in LDS

enum Mode { kRowFinal = 0, kChunkCand = 1, kCandFinal = 2 };

// Exclusive scan of one uint32 per wave (value taken from lane 0 of each
// wave) over the workgroup's 16 waves; returns this wave's offset, sets total.
__device__ __forceinline__ uint32_t wave_offsets(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t x = sh[w];
    off += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
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
__device__ __forceinline__ void find_bucket(const uint32_t* hist, int nbins, uint32_t k,
                                            uint32_t* scan_sh, uint32_t* sel_bin,
                                            uint32_t* sel_above) {
  const int per = nbins / kThreads;
  uint32_t c = 0;
  for (int q = 0; q < per; ++q) c += hist[nbins - 1 - per * threadIdx.x - q];
  // block exclusive scan of c in thread order (thread 0 = top bins)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  (void)lane;
  (void)wave;
  const uint32_t x = wave_inclusive_scan(c);
  uint32_t tot;
  const uint32_t woff = wave_offsets((uint32_t)__builtin_amdgcn_readlane((int)x, 63), scan_sh, tot);
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

template <int kMode>
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ logits, int64_t ld, const uint32_t* __restrict__ ckeys,
            const int32_t* __restrict__ cjs, int ncand, int chunk,
            const int32_t* __restrict__ row_len, const int32_t* __restrict__ row_seq,
            const int32_t* __restrict__ pt, int pt_stride, int c4_page_size,
            int32_t* __restrict__ phys_idx, int32_t* __restrict__ logical_idx,
            uint32_t* __restrict__ okeys, int32_t* __restrict__ ojs) {
  __shared__ uint32_t skey[kRegRow];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[2 * kWaves];
  __shared__ uint32_t sel_bin, sel_above;
  __shared__ uint32_t s_thr, s_need;  // threshold of a short bucket
  __shared__ uint32_t s_cand[kCandCap];  // keys of the threshold bucket

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
  } else {
    n = ncand;
  }
  const int K = min(kTopK, kMode == kCandFinal ? rl : n);  // entries to select
  const int E = (n + kThreads - 1) / kThreads;             // keys per lane (<= kMaxE)
  const int seg = wave * 64 * E;                           // first element of this wave

  // the histogram is cleared while the keys are in flight
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
  // keys in LDS; an element's index is base + e, or (candidates) re-read at
  // emission, which touches only the <= 512 selected ones
  const int nv = n - seg - lane;  // element i of this lane exists iff i < E and 64*i < nv
  {
    // batches of 8 unconditional loads (absent elements read element 0 of the
    // row and are dropped), so 8 loads per lane are in flight at once
    const float* lrow = logits + (int64_t)r * ld + base;
    const uint32_t* crow = ckeys + (int64_t)r * ncand;
    for (int i0 = 0; i0 < E; i0 += 8) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u;
        const bool ok = i < E && 64 * i < nv;
        const int e = ok ? seg + 64 * i + lane : 0;
        const uint32_t k = kMode == kCandFinal ? crow[e] : float_key(lrow[e]);
        kk[u] = ok ? k : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < E) skey[seg + 64 * (i0 + u) + lane] = kk[u];
    }
  }
  auto valid_at = [&](int i) { return i < E && 64 * i < nv; };
  auto key_at = [&](int i) { return skey[seg + 64 * i + lane]; };

  uint32_t thr = 0, need = 0;
  const bool take_all = n <= K;  // every element is selected
  if (!take_all) {
    // ---- 1. key range of the non-NaN keys
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = 0; i < E; ++i) {
      const uint32_t k = key_at(i);
      if (valid_at(i) && k != 0u) {
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    }
    kmin = wave_umin(kmin);
    kmax = wave_umax(kmax);
    if (lane == 0) {
      red[wave] = kmin;
      red[kWaves + wave] = kmax;
    }
    __syncthreads();
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
    for (int w = 0; w < kWaves; ++w) {
      kmin = min(kmin, red[w]);
      kmax = max(kmax, red[kWaves + w]);
    }
    if (kmin > kmax) kmin = kmax = 0u;  // every key is NaN
    const uint32_t range = kmax - kmin;
    const int sh = range == 0u ? 0 : max(0, (32 - __clz(range)) - 11);
    auto bin_of = [&](uint32_t k) -> uint32_t { return k == 0u ? 0u : 1u + ((k - kmin) >> sh); };

    // ---- 2. bucket of the K-th largest key
    for (int i = 0; i < E; ++i)
      if (valid_at(i)) atomicAdd(&hist[bin_of(key_at(i))], 1u);
    __syncthreads();
    find_bucket(hist, kBins, (uint32_t)K, red, &sel_bin, &sel_above);
    const uint32_t bstar = sel_bin;
    uint32_t k = (uint32_t)K - sel_above;

    // ---- 3. exact threshold inside the bucket (its keys share everything
    // above the low sh bits of key - kmin; NaN bucket 0 holds only key 0).
    // The bucket's members are gathered into a short LDS list when they fit.
    const uint32_t nb = hist[bstar];
    const bool listed = nb <= (uint32_t)kCandCap;
    __syncthreads();
    if (listed) {
      if (threadIdx.x == 0) sel_above = 0;  // reused as the list length
      __syncthreads();
      for (int i = 0; i < E; ++i) {
        const uint32_t kk = key_at(i);
        if (valid_at(i) && bin_of(kk) == bstar) s_cand[atomicAdd(&sel_above, 1u)] = kk;
      }
      __syncthreads();
    }
    uint32_t low = 0;  // threshold's low bits, built from the top
    int width = bstar == 0u ? 0 : sh;
    if (listed && nb <= (uint32_t)kThreads) {
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
      for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
      __syncthreads();
      if (listed) {
        for (int i = threadIdx.x; i < (int)nb; i += kThreads) {
          const uint32_t lo = (s_cand[i] - kmin) & ((1u << sh) - 1u);  // sh <= 21
          if ((lo & got_mask) == low) atomicAdd(&hist[(lo >> shift) & dmask], 1u);
        }
      } else {
        for (int i = 0; i < E; ++i) {
          const uint32_t kk = key_at(i);
          const uint32_t lo = (kk - kmin) & ((1u << sh) - 1u);
          const bool in = valid_at(i) && kk != 0u && bin_of(kk) == bstar && (lo & got_mask) == low;
          wave_hist_add(hist, (lo >> shift) & dmask, in);
        }
      }
      __syncthreads();
      find_bucket(hist, kBins, k, red, &sel_bin, &sel_above);
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

  // ---- 4. ordered placement: pos = #(key > thr before) + min(#(key == thr before), need)
  uint32_t gt_w = 0, eq_w = 0;
  for (int i = 0; i < E; ++i) {
    const bool v = valid_at(i);
    const uint32_t k = key_at(i);
    gt_w += (uint32_t)__popcll(__ballot(v && (take_all || k > thr)));
    eq_w += (uint32_t)__popcll(__ballot(v && !take_all && k == thr));
  }
  uint32_t tot;
  const uint32_t off = wave_offsets(gt_w | (eq_w << 16), red, tot);
  uint32_t g = off & 0xFFFFu, q = off >> 16;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int i = 0; i < E; ++i) {
    const bool v = valid_at(i);
    const uint32_t k = key_at(i);
    const bool isgt = v && (take_all || k > thr);
    const bool iseq = v && !take_all && k == thr;
    const uint64_t bg = __ballot(isgt), be = __ballot(iseq);
    const uint32_t gb = g + (uint32_t)__popcll(bg & lt);
    const uint32_t qb = q + (uint32_t)__popcll(be & lt);
    if (isgt || (iseq && qb < need)) {
      const uint32_t pos = gb + min(qb, need);
      const int e = seg + 64 * i + lane;
      const int j = kMode == kCandFinal ? cjs[(int64_t)r * ncand + e] : base + e;
      if (kMode == kChunkCand) {
        const int64_t o = ((int64_t)r * gridDim.x + blockIdx.x) * kTopK + pos;
        okeys[o] = k;
        ojs[o] = j;
      } else {
        phys_idx[(int64_t)r * kTopK + pos] =
            (int32_t)((int64_t)pt[(int64_t)row_seq[r] * pt_stride + j / c4_page_size] * c4_page_size +
                      j % c4_page_size);
        if (logical_idx) logical_idx[(int64_t)r * kTopK + pos] = j;
      }
    }
    g += (uint32_t)__popcll(bg);
    q += (uint32_t)__popcll(be);
  }
  // ---- padding
  for (int i = K + threadIdx.x; i < kTopK; i += kThreads) {
    if (kMode == kChunkCand) {
      const int64_t o = ((int64_t)r * gridDim.x + blockIdx.x) * kTopK + i;
      okeys[o] = 0u;
      ojs[o] = INT_MAX;
    } else {
      phys_idx[(int64_t)r * kTopK + i] = -1;
      if (logical_idx) logical_idx[(int64_t)r * kTopK + i] = -1;
    }
  }
}

int chunks_for(int64_t R, int64_t ld) {
  // enough chunks to put >= ~128 workgroups on the GPU, each within kRegRow
  int64_t want = (128 + R - 1) / R;
  int64_t c = (ld + want - 1) / want;
  c = std::max<int64_t>(c, 4096);
  c = std::min<int64_t>(c, kRegRow);
  int64_t chunks = (ld + c - 1) / c;
  if (chunks * kTopK > kRegRow) chunks = kRegRow / kTopK;  // candidates must fit one launch
  return (int)chunks;
}

}  // namespace

size_t topk_ws_bytes(int64_t R, int64_t max_len) {
  if (max_len <= kRegRow && (R >= 128 || max_len <= 8192)) return 0;
  const int chunks = chunks_for(R, max_len);
  return (size_t)R * chunks * kTopK * (sizeof(uint32_t) + sizeof(int32_t));
}

int64_t topk_max_len() { return (int64_t)(kRegRow / kTopK) * kRegRow; }

hipError_t launch_topk(const float* logits, int64_t ld, int R, const int32_t* row_len,
                       const int32_t* row_seq, const int32_t* page_table, int pt_stride,
                       int c4_page_size, int max_row_len, int32_t* phys_idx,
                       int32_t* logical_idx, void* ws, hipStream_t s) {
  (void)max_row_len;
  if (R == 0) return hipSuccess;
  if (ld <= kRegRow && (R >= 128 || ld <= 8192)) {
    hipLaunchKernelGGL(topk_kernel<kRowFinal>, dim3(1, R), dim3(kThreads), 0, s, logits, ld,
                       nullptr, nullptr, 0, 0, row_len, row_seq, page_table, pt_stride,
                       c4_page_size, phys_idx, logical_idx, nullptr, nullptr);
    return hipGetLastError();
  }
  const int chunks = chunks_for(R, ld);
  const int chunk = (int)((ld + chunks - 1) / chunks);
  uint32_t* ck = (uint32_t*)ws;
  int32_t* cj = (int32_t*)((uint8_t*)ws + (size_t)R * chunks * kTopK * sizeof(uint32_t));
  hipLaunchKernelGGL(topk_kernel<kChunkCand>, dim3(chunks, R), dim3(kThreads), 0, s, logits, ld,
                     nullptr, nullptr, 0, chunk, row_len, row_seq, page_table, pt_stride,
                     c4_page_size, nullptr, nullptr, ck, cj);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel<kCandFinal>, dim3(1, R), dim3(kThreads), 0, s, nullptr, 0, ck,
                     cj, chunks * kTopK, 0, row_len, row_seq, page_table, pt_stride,
                     c4_page_size, phys_idx, logical_idx, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace csa
