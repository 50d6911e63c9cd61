// indexer.hip -- lightning-indexer logits over the paged index-K pool.
//
// "Token 的一生：DSV4 架构与 DSpark" §3 (C4Indexer: FP8 or FP4 query and index-K,
// head weights fused with the query scale; §3.2 logits [bs, c4_seqlen] feed the
// top-512); "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）" CSA paragraph (a light,
// low-precision indexer scores every compressed block for each query).
//
//   logits[t][j] = sum_h w[t][h] * ReLU(qhat[t][h] . khat[j])
//
// Per query row the 64 heads share each index-K row, so scoring one entry is a
// [64 x 128] x [128] contraction: 16 KFLOP against 132 B (FP8) or 68 B (MXFP4)
// of index-K. At 8 TB/s that is ~1-2 PFLOP/s, beyond the fp32 vector units, so
// the scan runs on the gfx950 matrix cores: one v_mfma_scale_f32_16x16x128
// (FP8 e4m3, or MXFP4 with the e8m0 block scales applied by the instruction)
// scores 16 heads x 16 entries; four of them cover the 64 heads. Index-K rows
// stream from HBM straight into the B operand (each 16-entry group is one
// contiguous 2 KB / 1 KB read), the query sits in registers, and ReLU, the
// head weights and the 64-head reduction run in the epilogue on the
// accumulators.
#include <limits.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "topk_select.hpp"
#include "wave_topk.hpp"

namespace csa {
namespace {

constexpr int kHeads = 64;   // indexer heads handled by the MFMA path
constexpr int kDim = 128;    // indexer head dim handled by the MFMA path
constexpr int kWaves = 4;
constexpr int kRing = 2;     // 64-entry batches in flight per wave
constexpr int kWgEntries = kWaves * kRing * 64;
constexpr int kMaxChunk = 8 * kWgEntries;  // entries per workgroup, at most
constexpr int kScanSlots = 256;            // scan workgroups resident at once (one per CU)
// Long ragged batches (more entries than kScanSlots chunks of 4096, at most
// kWideRows rows): the scan takes chunks of up to kWideChunk entries, their
// length and the work items planned on the device from the rows' lengths
// (wide_item).
constexpr int kWideChunk = kMaxChunk + 2 * kWgEntries;
constexpr int kWideRows = 256;

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, v4f c) {
  // format 0 = FP8 e4m3 for both operands; e8m0 scale 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ v4f mfma_fp4(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  // format 4 = FP4 e2m1 for both operands (low 4 registers used); per-lane e8m0 scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// Operand layout of v_mfma_*_16x16x128 (64 lanes): lane l supplies row / column
// (l % 16) and the 32 K-elements [(l/16)*32, (l/16)*32 + 32) of it; with MXFP4
// that K-range is one 32-element scale block, whose e8m0 byte the lane
// supplies as its scale. The result lane l holds rows 4*(l/16) + 0..3 of
// column l % 16.
//
// kCand: instead of the logits, the workgroup writes its chunk's top-512
// candidates (order-preserving keys and entry indices, in index order; a chunk
// past the row writes padding: key 0, index INT_MAX), selected from the logits
// in LDS exactly as the top-512 kernel's chunk pass selects them from memory.
// Any entry of a row's top-512 is in its chunk's top-512, so the top-512 of the
// candidates is the row's. The kCand workgroup has kSelWaves waves: the first
// kScanWaves scan, all of them select (fewer keys per lane, the same barriers).
constexpr int kSelWaves = 8;
template <bool kCand>
constexpr int idx_threads() { return (kCand ? kSelWaves : kWaves) * 64; }
// Scan waves: kWaves, or (MXFP4 with the selection) all kSelWaves: an MXFP4
// row is half as many bytes for the same matrix and epilogue work per entry,
// so its scan is bound by the latency of that work more than by HBM, and a
// second wave per SIMD hides it.
template <bool kFp4, bool kCand>
constexpr int kScanWaves() { return kFp4 && kCand ? kSelWaves : kWaves; }

// Candidate lists that one workgroup of the scan writes and another reads in
// the same launch go around the caches: the eight XCDs' L2 caches are not
// coherent with each other, and making them so with a device-scope fence costs
// a write-back of the whole L2 per workgroup. System-scope stores write
// through to memory and system-scope loads read from it; the writer waits for
// its stores to complete (vmcnt 0) before it counts itself in.
template <class T>
__device__ __forceinline__ void st_through(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <class T>
__device__ __forceinline__ T ld_through(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Top-K of n <= kTH * kE candidates (keys, entry indices, slots; in index
// order) by one workgroup, emitted either as a candidate list (out_keys /
// out_js / out_phys: 512 entries, padding past K: key 0, index INT_MAX, slot
// -1) or as the row's selection (phys_idx / logical_idx: 512 entries, -1
// past K). L.hist must be clear; ends with the emission (no barrier).
template <int kTH, int kE>
__device__ __forceinline__ void cand_select_emit(const uint32_t* keys, const int32_t* js,
                                                 const int32_t* phys, int n, int K, TopkLds& L,
                                                 uint32_t* out_keys, int32_t* out_js,
                                                 int32_t* out_phys, int32_t* phys_idx,
                                                 int32_t* logical_idx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = wave * 64 * kE;
  // keys, entry indices and slots in one round of loads; the selected ones'
  // indices and slots are parked beside them
  uint32_t kr[kE];
  int32_t ja[kE], pa[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int e = seg + 64 * i + lane;
    const bool ok = e < n;
    kr[i] = ok ? ld_through(keys + e) : 0u;
    ja[i] = ok ? ld_through(js + e) : -1;
    pa[i] = ok ? ld_through(phys + e) : -1;
  }
  topk_select_pay<kE, kTH>(kr, ja, pa, n, K, seg, L);
  for (int p = threadIdx.x; p < kTopK; p += kTH) {
    const int32_t ph = p < K ? topk_pay_b(L)[p] : -1;
    const int32_t jj = p < K ? topk_pay_a(L)[p] : -1;
    if (phys_idx) {
      phys_idx[p] = ph;
      if (logical_idx) logical_idx[p] = jj;
    } else {
      st_through(out_keys + p, p < K ? L.out_k[p] : 0u);
      st_through(out_js + p, p < K ? jj : (int32_t)INT_MAX);
      st_through(out_phys + p, ph);
    }
  }
}

// Counts this workgroup in at *c once every thread's write-through stores have
// completed; true in every thread of the workgroup that brings the count to
// `members`, which also returns the counter to zero.
__device__ __forceinline__ bool last_arrival(uint32_t* c, int members, int* s_flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    // system scope: performed at memory, where every XCD's workgroups meet
    const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const bool last = old + 1u == (uint32_t)members;
    if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// The finish of the fused selection, run by every scan workgroup whose chunk
// holds entries of the row (`live` such chunks, the first ones) after it has
// written its chunk's candidates: the last workgroup of its group of chunks
// merges the group (or, when the row's live chunks form one group, selects
// the row); the last group of the row selects the row from the groups' lists.
template <int kTH, int kE>
__device__ __forceinline__ void cand_finish(const CandOut& co, int t, int x, int nch, int rl,
                                            int live, TopkLds& L) {
  __shared__ int s_flag;
  const int g = x / co.gsize;
  const int members = min(co.gsize, live - g * co.gsize);
  const int groups = (live + co.gsize - 1) / co.gsize;
  uint32_t* const cnt = co.cnt + (int64_t)t * (kCandGroups + 1);
  if (!last_arrival(cnt + g, members, &s_flag)) return;
  for (int i = threadIdx.x; i < kTopkBins; i += kTH) L.hist[i] = 0u;
  const int64_t cb = ((int64_t)t * nch + (int64_t)g * co.gsize) * kTopK;
  const int n1 = members * kTopK;
  if (groups == 1) {
    cand_select_emit<kTH, kE>(co.keys + cb, co.js + cb, co.phys + cb, n1, min(kTopK, rl), L,
                              nullptr, nullptr, nullptr, co.phys_idx + (int64_t)t * kTopK,
                              co.logical_idx ? co.logical_idx + (int64_t)t * kTopK : nullptr);
    return;
  }
  const int64_t mb = ((int64_t)t * co.ngroups + g) * kTopK;
  cand_select_emit<kTH, kE>(co.keys + cb, co.js + cb, co.phys + cb, n1, min(kTopK, n1), L,
                            co.mkeys + mb, co.mjs + mb, co.mphys + mb, nullptr, nullptr);
  if (!last_arrival(cnt + kCandGroups, groups, &s_flag)) return;
  for (int i = threadIdx.x; i < kTopkBins; i += kTH) L.hist[i] = 0u;
  const int64_t rb = (int64_t)t * co.ngroups * kTopK;
  cand_select_emit<kTH, kE>(co.mkeys + rb, co.mjs + rb, co.mphys + rb, groups * kTopK,
                            min(kTopK, rl), L, nullptr, nullptr, nullptr,
                            co.phys_idx + (int64_t)t * kTopK,
                            co.logical_idx ? co.logical_idx + (int64_t)t * kTopK : nullptr);
}

// The scan over a long ragged batch (indexer_wide_kernel): workgroup j takes work item j
// (the grid has one workgroup per 4096-entry chunk slot of every row, at
// least as many as there are items; those past the last item exit). The chunk
// length is chosen from the rows' lengths: of 4096, 4608 and 5120 entries,
// the one whose live chunks, taken kScanSlots at a time, scan the fewest
// entries per workgroup slot (rounds x length; ties to the shorter). The
// items are first every row's live chunks, row after row (an empty row whose
// selection finishes in the scan counts one, where its empty selection is
// written), then, when the candidates go to the final pass, the rows'
// remaining chunk slots (their padding is written). Consecutive items go to
// consecutive workgroups and so round-robin over the XCDs: the live chunks
// spread evenly over them whatever the rows' lengths, and the workgroups with
// no item come after all of them. Every workgroup computes the same plan
// from the same row lengths (rows 64 k + lane are this lane's, k < 4: at most
// kWideRows rows) and takes from it item j: its row t and chunk slot x, the
// chunk length, and the number of items (j >= total: none).
template <int kBlocks>
__device__ __forceinline__ void wide_item_k(const int32_t* __restrict__ row_len, int T, int nch,
                                            bool fused, int j, int& t, int& x, int& chunk,
                                            int& total, int& n_t) {
  const int lane = threadIdx.x & 63;
  int n[kBlocks];
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) {
    const int r = 64 * k + lane;
    n[k] = r < T ? max(row_len[r], 0) : 0;
  }
  // live chunks per row for each candidate length (divisions by constants)
  int cnt[3][kBlocks];
  int vbest = 0;
  uint64_t best_cost = ~0ull;
#pragma unroll
  for (int v = 0; v < 3; ++v) {
    constexpr int kLen0 = kMaxChunk;
    const uint32_t len = kLen0 + v * kWgEntries;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kBlocks; ++k) {
      cnt[v][k] = (int)(((uint32_t)n[k] + len - 1) / len);
      c += (uint32_t)cnt[v][k];
    }
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(c), 63);
    const uint64_t cost = (uint64_t)((tot + kScanSlots - 1) / kScanSlots) * len;
    if (cost < best_cost) {
      best_cost = cost;
      vbest = v;
    }
  }
  chunk = kMaxChunk + vbest * kWgEntries;
  // items of the first kind (live chunks; an empty row's one) and of the
  // second (the remaining slots) per row, and their inclusive prefixes
  int lv[kBlocks], a[kBlocks], ai[kBlocks], bi[kBlocks];
  int ca = 0, cb = 0;
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) {
    const bool in = 64 * k + lane < T;
    lv[k] = min(vbest == 0 ? cnt[0][k] : vbest == 1 ? cnt[1][k] : cnt[2][k], nch);
    a[k] = in ? (fused && n[k] == 0 ? 1 : lv[k]) : 0;
    const int sa = (int)wave_inclusive_scan((uint32_t)a[k]);
    ai[k] = ca + sa;
    ca += __builtin_amdgcn_readlane(sa, 63);
    if (!fused) {
      const int sb = (int)wave_inclusive_scan((uint32_t)(in ? nch - lv[k] : 0));
      bi[k] = cb + sb;
      cb += __builtin_amdgcn_readlane(sb, 63);
    } else {
      bi[k] = 0;
    }
  }
  total = ca + cb;
  t = 0;
  x = 0;
  n_t = 0;
  if (j >= total) return;
  const bool second = j >= ca;
  const int d = second ? j - ca : j;
#pragma unroll
  for (int k = 0; k < kBlocks; ++k) {
    const int inc = second ? bi[k] : ai[k];
    const uint64_t m = __ballot(inc > d);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;  // the first row whose items reach past d
      const int lvl = __builtin_amdgcn_readlane(lv[k], l);
      const int cnt_l = second ? nch - lvl : __builtin_amdgcn_readlane(a[k], l);
      const int excl = __builtin_amdgcn_readlane(inc, l) - cnt_l;
      t = 64 * k + l;
      x = (second ? lvl : 0) + d - excl;
      n_t = __builtin_amdgcn_readlane(n[k], l);
      return;
    }
  }
}

__device__ __forceinline__ void wide_item(const int32_t* __restrict__ row_len, int T, int nch,
                                          bool fused, int j, int& t, int& x, int& chunk,
                                          int& total, int& n_t) {
  if (T <= 64) wide_item_k<1>(row_len, T, nch, fused, j, t, x, chunk, total, n_t);
  else wide_item_k<4>(row_len, T, nch, fused, j, t, x, chunk, total, n_t);
}

// One scan work item: chunk slot x (entries x * chunk ..) of row t, of
// length n, whose candidates or logits sit in slot x of nch per row.
template <bool kFp4, bool kPage64, bool kCand, int kCap>
__device__ __forceinline__ void scan_chunk_item(
    int t, int x, int nch, int chunk, int n, const uint8_t* __restrict__ qc, const void* __restrict__ qs,
    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ pt, int pt_stride,
    const uint8_t* __restrict__ kdata, const void* __restrict__ kscale, int page_size,
    float* __restrict__ logits, int64_t ld, const CandOut& co) {
  constexpr int kRowBytes = kFp4 ? kDim / 2 : kDim;  // bytes per index-K / q row
  constexpr int kTH = idx_threads<kCand>();
  constexpr int kSelE = kCap / kTH;      // keys per lane of the chunk's selection
  constexpr int kFinE = kMaxChunk / kTH;  // and of the finish (at most 8 x 512 candidates)
  constexpr int kSW = kScanWaves<kFp4, kCand>();  // waves that scan
  __shared__ int32_t s_pages[kCap / 16 + 2];      // physical pages of this chunk
  __shared__ __attribute__((aligned(16))) float s_out[kCap + 64];  // the chunk's logits
  __shared__ TopkLds L;                                  // the selections (kCand)
  const int c0 = x * chunk;
  // chunks holding entries of the row (a row longer than the call's bound
  // is cut at nch chunks, as the grid covers no more)
  const int live = min((n + chunk - 1) / chunk, nch);
  if (c0 >= n) {
    if constexpr (kCand) {
      if (co.ngroups > 0) {
        // past the row: no part in the fused finish; an empty row's selection
        // is written here
        if (n == 0 && x == 0)
          for (int p = threadIdx.x; p < kTopK; p += kTH) {
            co.phys_idx[(int64_t)t * kTopK + p] = -1;
            if (co.logical_idx) co.logical_idx[(int64_t)t * kTopK + p] = -1;
          }
      } else {
        for (int p = threadIdx.x; p < kTopK; p += kTH) {
          const int64_t o = ((int64_t)t * nch + x) * kTopK + p;
          co.keys[o] = 0u;
          co.js[o] = INT_MAX;
          co.phys[o] = -1;
        }
      }
    }
    return;
  }
  const int c1 = min(c0 + chunk, n);
  const int seq = row_seq[t];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop
  const int col = lane & 15;
  const int grp = lane >> 4;

  // Page ids of the chunk, once: the scan below then issues its index-K loads
  // without waiting on page-table reads.
  const int32_t* ptrow = pt + (int64_t)seq * pt_stride;
  const int pg0 = c0 / page_size;
  const int npg = (c1 - 1) / page_size - pg0 + 1;
  for (int i = threadIdx.x; i < npg; i += idx_threads<kCand>()) s_pages[i] = ptrow[pg0 + i];

  if (kCand && wave >= kSW) {
    __syncthreads();  // the page ids (the scan waves pass the same barrier)
  } else {
  // Query operands: head hb*16 + col, K-elements grp*32 .. grp*32+31.
  v8i a[4];
  int sa[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = hb * 16 + col;
    const uint8_t* p = qc + ((int64_t)t * kHeads + head) * kRowBytes + grp * (kRowBytes / 4);
    if (kFp4) {
      uint4 x = *reinterpret_cast<const uint4*>(p);
      a[hb] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      sa[hb] = reinterpret_cast<const uint8_t*>(qs)[((int64_t)t * kHeads + head) * 4 + grp];
    } else {
      uint4 x = *reinterpret_cast<const uint4*>(p);
      uint4 y = *reinterpret_cast<const uint4*>(p + 16);
      a[hb] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      sa[hb] = 127;
    }
  }
  // Head weights for the accumulator rows this lane holds (FP8: q scale folded
  // in, valid because ReLU(s x) = s ReLU(x) for s > 0).
  float wq[16];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hb * 16 + grp * 4 + r;
      float v = w[(int64_t)t * kHeads + h];
      if (!kFp4) v *= reinterpret_cast<const float*>(qs)[(int64_t)t * kHeads + h];
      wq[hb * 4 + r] = v;
    }
  __syncthreads();

  // Entries go in batches of 64 (four 16-entry groups; a group never
  // straddles a page since page_size % 16 == 0 and the chunk starts on a
  // multiple of 16, so its page is wave-uniform). Wave w takes batches w,
  // w + kWaves, ... and keeps kR batches of loads in flight (a register
  // ring, slot = batch % kR). After the 16 MFMAs of a batch, one
  // reduce-scatter across the four lane rows leaves in row r the 64-head sum
  // of group r, so each lane stores one logit and a wave writes the batch's
  // 64 logits as one contiguous 256-byte store; the lane also loads the FP8
  // scale of exactly that entry. The logits collect in LDS and are written
  // out after the loop: a global store inside it would sit in the same
  // in-order memory counter as the loads and delay every later wait. The loop
  // is branch-free: batches past the chunk load entry 0 of its first page (or
  // their page), and their logits land in LDS past the chunk and are dropped.
  const int nbatch = (c1 - c0 + 63) / 64;
  const int nb = (nbatch - wave + kSW - 1) / kSW;  // batches of this wave
  constexpr int kR = kRing;  // (measured on the MXFP4 scan at 1M: a 4-batch ring is slower)
  v8i b[kR][4];
  int sb[kR][4];
  float ks[kR];
  auto slot_of = [&](int j, int g0) __attribute__((always_inline)) {
    const int pg = s_pages[g0 < c1 ? g0 / page_size - pg0 : 0];
    return (j < c1) ? (int64_t)pg * page_size + j % page_size : (int64_t)s_pages[0] * page_size;
  };
  // 64-entry pages (the C4 layout): a batch is one page (the chunk starts on a
  // page), found with no division; entries past the chunk read their page
  // anyway (their logits are dropped)
  const int last_pg = npg - 1;
  auto batch_page = [&](int i) __attribute__((always_inline)) {
    return (int64_t)s_pages[min(i * kSW + wave, last_pg)] * 64;
  };
  auto issue = [&](int i, auto R) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    const int e0 = c0 + (i * kSW + wave) * 64;  // first entry of the batch
    const int64_t pbase = kPage64 ? batch_page(i) : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int g0 = e0 + 16 * k;
      const int64_t slot = kPage64 ? pbase + 16 * k + col : slot_of(g0 + col, g0);
      const uint8_t* p = kdata + slot * kRowBytes + grp * (kRowBytes / 4);
      if (kFp4) {
        const v4i x = *reinterpret_cast<const v4i*>(p);
        b[r][k] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        // the entry's four block-scale bytes as one word; the lane's byte is
        // taken at the use (a byte load would be narrowed and re-extended at
        // the loop head, where it waits for every outstanding load)
        sb[r][k] = reinterpret_cast<const int32_t*>(kscale)[slot];
      } else {
        const v4i x = *reinterpret_cast<const v4i*>(p);
        const v4i y = *reinterpret_cast<const v4i*>(p + 16);
        b[r][k] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        sb[r][k] = 127;
      }
    }
    if (!kFp4) {  // scale of the entry this lane stores: group grp, column col
      const int g0 = e0 + 16 * grp;
      const int64_t slot = kPage64 ? pbase + 16 * grp + col : slot_of(g0 + col, g0);
      ks[r] = reinterpret_cast<const float*>(kscale)[slot];
    } else {
      ks[r] = 1.f;
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads together, in issue order
  };
  auto step = [&](int i, auto R, auto Last) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    float pk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v4f acc[4];
      const int sbk = kFp4 ? (int)__builtin_amdgcn_ubfe((uint32_t)sb[r][k], 8 * grp, 8) : 127;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        acc[hb] = kFp4 ? mfma_fp4(a[hb], b[r][k], v4f{0.f, 0.f, 0.f, 0.f}, sa[hb], sbk)
                       : mfma_fp8(a[hb], b[r][k], v4f{0.f, 0.f, 0.f, 0.f});
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int q = 0; q < 4; ++q) v = fmaf(wq[hb * 4 + q], fmaxf(acc[hb][q], 0.f), v);
      pk[k] = v;
    }
    const float tot = rows4_reduce_scatter(pk[0], pk[1], pk[2], pk[3]);
    // entry within the chunk; a batch past this wave's last lands in the
    // spare 64 slots at the end
    const int jl = i < nb ? (i * kSW + wave) * 64 + 16 * grp + col : kCap + lane;
    s_out[jl] = tot * ks[r];
    // refill the slot just consumed. In the last round of the loop no load
    // goes past this wave's last batch (a step past it reads stale registers
    // and drops its logits), so none is still in flight when the selection
    // reuses the registers; the main loop's refills stay unconditional (a
    // branch there makes the compiler drain every load before it).
    if constexpr (decltype(Last)::value) {
      if (i + kR < nb) issue(i + kR, R);
    } else {
      issue(i + kR, R);
    }
  };
  static_assert(kR == 2 || kR == 4, "the batch loop below is unrolled by hand for 2 or 4 slots");
  if (0 < nb) issue(0, std::integral_constant<int, 0>{});
  if (1 < nb) issue(1, std::integral_constant<int, 1>{});
  if constexpr (kR == 4) {
    if (2 < nb) issue(2, std::integral_constant<int, 2>{});
    if (3 < nb) issue(3, std::integral_constant<int, 3>{});
  }
  using std::integral_constant;
  const integral_constant<bool, false> body;
  const integral_constant<bool, true> last;
  int i0 = 0;
  for (; i0 + 2 * kR <= nb; i0 += kR) {  // every refill is a batch of this wave
    step(i0, integral_constant<int, 0>{}, body);
    step(i0 + 1, integral_constant<int, 1>{}, body);
    if constexpr (kR == 4) {
      step(i0 + 2, integral_constant<int, 2>{}, body);
      step(i0 + 3, integral_constant<int, 3>{}, body);
    }
  }
  for (; i0 < nb; i0 += kR) {
    step(i0, integral_constant<int, 0>{}, last);
    step(i0 + 1, integral_constant<int, 1>{}, last);
    if constexpr (kR == 4) {
      step(i0 + 2, integral_constant<int, 2>{}, last);
      step(i0 + 3, integral_constant<int, 3>{}, last);
    }
  }
  }  // scan waves
  __syncthreads();
  const int n_out = c1 - c0;
  if constexpr (kCand) {
    // keys from LDS: element seg + 64 i + lane of this wave's segment
    constexpr int kE = kSelE;
    for (int i = threadIdx.x; i < kTopkBins; i += kTH) L.hist[i] = 0u;
    const int seg = wave * 64 * kE;
    // all of the lane's logits loaded at once (e < kCap: in bounds), then
    // keyed; the empty asm keeps the compiler from sinking each load into a
    // branch of its own, one LDS round trip after another
    float v[kE];
#pragma unroll
    for (int i = 0; i < kE; ++i) v[i] = s_out[seg + 64 * i + lane];
#pragma unroll
    for (int i = 0; i < kE; ++i) asm volatile("" : "+v"(v[i]));
    uint32_t kr[kE];
#pragma unroll
    for (int i = 0; i < kE; ++i)  // masked, not branched: key 0 past the chunk
      kr[i] = float_key(v[i]) & (0u - (uint32_t)(seg + 64 * i + lane < n_out));
    const int K = min(kTopK, n_out);
    topk_select<kE, kTH>(kr, n_out, K, seg, L);
    for (int p = threadIdx.x; p < kTopK; p += kTH) {
      const int64_t o = ((int64_t)t * nch + x) * kTopK + p;
      uint32_t key = 0u;  // padding past K
      int32_t j = INT_MAX, phys = -1;
      if (p < K) {
        key = L.out_k[p];
        j = c0 + L.out_e[p];
        phys = s_pages[j / page_size - pg0] * page_size + j % page_size;  // a page of this chunk
      }
      if (co.ngroups > 0) {  // read by another workgroup of this launch
        st_through(co.keys + o, key);
        st_through(co.js + o, j);
        st_through(co.phys + o, phys);
      } else {
        co.keys[o] = key;
        co.js[o] = j;
        co.phys[o] = phys;
      }
    }
    if (co.ngroups > 0) cand_finish<kTH, kFinE>(co, t, x, nch, n, live, L);
  } else {
    float* orow = logits + (int64_t)t * ld + c0;
    for (int j = threadIdx.x; j < n_out; j += kWaves * 64) orow[j] = s_out[j];
  }
}

// The decode scan: workgroup (x, t) takes chunk x of row t.
template <bool kFp4, bool kPage64, bool kCand>
__global__ void __launch_bounds__(idx_threads<kCand>())
indexer_mfma_kernel(const uint8_t* __restrict__ qc, const void* __restrict__ qs,
                    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ row_len, const int32_t* __restrict__ pt,
                    int pt_stride, const uint8_t* __restrict__ kdata,
                    const void* __restrict__ kscale, int page_size, float* __restrict__ logits,
                    int64_t ld, int chunk, CandOut co) {
  scan_chunk_item<kFp4, kPage64, kCand, kMaxChunk>(blockIdx.y, blockIdx.x, gridDim.x, chunk,
                                                   row_len[blockIdx.y], qc, qs, w, row_seq, pt,
                                                   pt_stride, kdata, kscale, page_size, logits, ld,
                                                   co);
}

// The decode scan of a long ragged batch (64-entry pages, fused selection):
// workgroup j takes item j of the plan of wide_item, over co.wide_rows rows
// of co.wide_chunks chunk slots.
template <bool kFp4>
__global__ void __launch_bounds__(idx_threads<true>())
indexer_wide_kernel(const uint8_t* __restrict__ qc, const void* __restrict__ qs,
                    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ row_len, const int32_t* __restrict__ pt,
                    int pt_stride, const uint8_t* __restrict__ kdata,
                    const void* __restrict__ kscale, CandOut co) {
  int t, x, ch, total, n;
  wide_item(row_len, co.wide_rows, co.wide_chunks, co.ngroups > 0, (int)blockIdx.x, t, x, ch,
            total, n);
  if ((int)blockIdx.x >= total) return;
  scan_chunk_item<kFp4, true, true, kWideChunk>(t, x, co.wide_chunks, ch, n, qc, qs, w, row_seq,
                                                pt, pt_stride, kdata, kscale, 64, nullptr, 0, co);
}

// Many query rows of few sequences (prefill; multi-token decode, whose rows
// come in groups that share a sequence): a workgroup of 8 waves owns kRows
// consecutive rows (2..8; each row's 64 heads in registers, a row shared by
// 8 / kRows waves that split each page's four 16-entry groups, the waves past
// kRows * (8 / kRows) only stage) and walks a
// range of the index-K pages of their sequence once: each 64-entry page is
// staged into LDS with one coalesced 16-byte load per thread (double-buffered,
// 16-byte chunks XOR-swizzled by entry so the MFMA operand reads are
// conflict-free) and scored by all the rows, so index-K is read once per
// kRows rows instead of once per row. blockIdx.y picks the range (pages
// [y * ppc, (y + 1) * ppc)), so that a few row groups still fill the chip. Row
// ends (the causal rule) are enforced by per-row buffer stores bounded to
// row_len. A row of another sequence than the workgroup's first row reads its
// own pages straight from memory.
//
// kSel (8 rows, one wave per row): no logits are written. Each wave keeps the
// running top-512 of its row's logits in LDS as they are produced (WaveTopk:
// a candidate buffer and a rising threshold), and at the end writes either the
// row's selection (one page range: physical slots through the page table and
// entry indices, as the top-512 kernel writes them) or its range's top-512
// candidates (key, index, slot; key 0 / INT_MAX / -1 padding) for the final
// pass over the ranges. Any entry of the row's top-512 is in its range's
// top-512, so the result is exact.
constexpr int kRowsPerWG = 8;  // waves per workgroup (and rows, at most)
constexpr int kSelCap = 1024;  // per-row candidate buffer of the fused selection
constexpr int kSelSpan = 65536;  // entries per page range, at most (16-bit offsets in the buffer)

template <bool kFp4, int kRows, bool kSel>
__global__ void __launch_bounds__(kRowsPerWG * 64) __attribute__((amdgpu_waves_per_eu(4)))
indexer_rows_kernel(const uint8_t* __restrict__ qc, const void* __restrict__ qs,
                    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ row_len, int T, const int32_t* __restrict__ pt,
                    int pt_stride, const uint8_t* __restrict__ kdata,
                    const void* __restrict__ kscale, float* __restrict__ logits, int64_t ld,
                    int ppc, CandOut co) {
  static_assert(kRows >= 2 && kRows <= kRowsPerWG, "rows per workgroup");
  // waves per row: with the fused selection one (its running top-512 belongs
  // to one wave; the waves past kRows only stage), else 8 / kRows
  constexpr int kWpr = kSel ? 1 : kRowsPerWG / kRows;
  constexpr int kPage = 64;                          // entries per page (= tile)
  constexpr int kRowBytes = kFp4 ? kDim / 2 : kDim;  // bytes per index-K row
  constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kPage * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_bs[2][kPage];  // fp32 scale / 4 e8m0 bytes
  __shared__ int s_len[kRows];
  // fused selection: per wave, candidate keys, 16-bit index offsets and a
  // 256-bin histogram; s_cflag[i]: some wave asks every wave to compact at the
  // next page of slot i (so that the waves' compactions overlap instead of
  // each one holding the workgroup at the next page's barrier)
  constexpr int kSelWords = kSelCap + kSelCap / 2 + 256;
  __shared__ __attribute__((aligned(16))) uint32_t s_sel[kSel ? kRowsPerWG * kSelWords : 4];
  __shared__ int s_cflag[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps the row state scalar
  const int sub = wave % kWpr;  // this wave scores the groups g with g % kWpr == sub
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int t0 = blockIdx.x * kRows;
  const int t = t0 + wave / kWpr;
  const bool live = wave < kRows * kWpr;  // the other waves only stage
  const bool row_ok = live && t < T;
  const int seq0 = row_seq[t0];
  const int seqw = row_ok ? row_seq[t] : seq0;
  const bool own = seqw == seq0;
  const int nw = row_ok ? row_len[t] : 0;
  if (lane == 0 && sub == 0 && live) s_len[wave / kWpr] = own ? nw : -nw - 1;  // other sequence: negated
  WaveTopk<kSelCap, kTopK> sel;
  if constexpr (kSel) {
    sel.key = s_sel + wave * kSelWords;
    sel.idx = reinterpret_cast<uint16_t*>(sel.key + kSelCap);
    sel.hist = sel.key + kSelCap + kSelCap / 2;
    if (tid < 3) s_cflag[tid] = 0;  // ordered before use by the barrier below
  }

  // query operands and head weights of this wave's row
  v8i a[4];
  int sa[4];
  float wq[16];
  const int tq = row_ok ? t : t0;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = hb * 16 + col;
    const uint8_t* p = qc + ((int64_t)tq * kHeads + head) * kRowBytes + grp * (kRowBytes / 4);
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    if (kFp4) {
      a[hb] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      sa[hb] = reinterpret_cast<const uint8_t*>(qs)[((int64_t)tq * kHeads + head) * 4 + grp];
    } else {
      const uint4 y = *reinterpret_cast<const uint4*>(p + 16);
      a[hb] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      sa[hb] = 127;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = hb * 16 + grp * 4 + r;
      float v = w[(int64_t)tq * kHeads + h];
      if (!kFp4) v *= reinterpret_cast<const float*>(qs)[(int64_t)tq * kHeads + h];
      wq[hb * 4 + r] = v;
    }
  }
  __syncthreads();
  int maxown = 0, maxall = 0;  // staging covers the first sequence's rows only
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int v = s_len[i];
    maxown = max(maxown, v);
    maxall = max(maxall, v >= 0 ? v : -v - 1);
  }
  // this workgroup's page range [pc0, pc1)
  const int pc0 = blockIdx.y * ppc, pc1 = pc0 + ppc;
  const int jbase = pc0 * kPage;  // the selection buffer holds entry - jbase
  const int npages = min((maxall + kPage - 1) / kPage, pc1);
  const int nstage = min((maxown + kPage - 1) / kPage, pc1);
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      kSel ? nullptr : logits + (int64_t)tq * ld, (short)0, kSel ? 0 : nw * 4, 0x00020000);
  const int32_t* pt0 = pt + (int64_t)seq0 * pt_stride;
  const int32_t* ptw = pt + (int64_t)seqw * pt_stride;

  // staging: thread i < kPage*kChunks moves chunk (i % kChunks) of entry i / kChunks.
  // Every thread issues the loads (spare threads duplicate a chunk) so that
  // the loop holds no conditional load and outstanding loads stay countable.
  const bool stager = tid < kPage * kChunks;
  const int stid = tid % (kPage * kChunks);
  const int se = stid / kChunks, sc = stid % kChunks;
  const int sw = kFp4 ? (sc ^ ((se >> 2) & 3)) : (sc ^ (se & 7));  // swizzled chunk position
  const bool scaler = tid < kPage;  // one wave also moves the page's 256 B of scales
  const int sce = tid % kPage;        // the entry whose 4 scale bytes this thread moves
  // pages are loaded kDepth pages ahead into a register ring (slot p % kDepth)
  constexpr int kDepth = 3;
  v4i stage[kDepth];  // native vectors (HIP's uint4 struct blocks promotion)
  uint32_t sstage[kDepth];
  auto load_page = [&](int p, auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    // clamped, never skipped; with no page to stage, pool page 0 stands in
    const int64_t base = nstage > 0 ? (int64_t)pt0[min(p, nstage - 1)] * kPage : 0;
    stage[k] = *reinterpret_cast<const v4i*>(kdata + (base + se) * kRowBytes + sc * 16);
    sstage[k] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(kscale) + (base + sce) * 4);
  };
  // issue order fixed (slot 0 oldest) so the loop head waits only for slot 0
  load_page(pc0, std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  load_page(pc0 + 1, std::integral_constant<int, 1>{});
  __builtin_amdgcn_sched_barrier(0);
  load_page(pc0 + 2, std::integral_constant<int, 2>{});
  __builtin_amdgcn_sched_barrier(0);
  // 64 heads x 16 entries: 4 MFMAs, ReLU, head weights, 64-head reduction,
  // logit store (lanes of rows past their row_len are dropped by the buffer)
  // ReLU and head weights of one 16-entry group, summed over this lane's 16
  // heads (the other heads of the entry are in the other lane rows)
  // (a wave issuing its matrix ops runs at raised priority, so that the
  // matrix cores are fed first and the other waves' epilogues fill the gaps:
  // prefill 1187 -> 1129 us)
  auto head_sum = [&](const v8i& bb, int sb) __attribute__((always_inline)) {
    v4f acc[4];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      acc[hb] = kFp4 ? mfma_fp4(a[hb], bb, v4f{0.f, 0.f, 0.f, 0.f}, sa[hb], sb)
                     : mfma_fp8(a[hb], bb, v4f{0.f, 0.f, 0.f, 0.f});
    __builtin_amdgcn_s_setprio(0);
    float v = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) v = fmaf(wq[hb * 4 + r], fmaxf(acc[hb][r], 0.f), v);
    return v;
  };
  auto score_store = [&](const v8i& bb, int sb, float ks, int jrow) __attribute__((always_inline)) {
    v4f acc[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      acc[hb] = kFp4 ? mfma_fp4(a[hb], bb, v4f{0.f, 0.f, 0.f, 0.f}, sa[hb], sb)
                     : mfma_fp8(a[hb], bb, v4f{0.f, 0.f, 0.f, 0.f});
    float v = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) v = fmaf(wq[hb * 4 + r], fmaxf(acc[hb][r], 0.f), v);
    v = cross_row_sum(v);
    if constexpr (kSel) {
      sel.push(v * ks, (uint32_t)(jrow - jbase), grp == 0 && jrow < nw);
    } else {
      const int off = grp == 0 ? jrow * 4 : 0x7FFFFFFF;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v * ks), out_rsrc, off, 0, 0);
    }
  };
  auto page_step = [&](const int p, auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    const int buf = p & 1;
    if (stager) *reinterpret_cast<v4i*>(&s_b[buf][se * kRowBytes + sw * 16]) = stage[k];
    if (scaler) s_bs[buf][sce] = sstage[k];
    __syncthreads();
    load_page(p + kDepth, K);  // refill the slot just written to LDS
    // a compaction asked for at the previous page: every wave with more than
    // 512 candidates compacts at this one, together, before its push (the
    // flag is read here and used after the scoring, which hides the read);
    // the flag read one page ago is cleared (its readers have all passed this
    // page's barrier)
    int cflag = 0;
    if constexpr (kSel) {
      cflag = s_cflag[k];
      if (tid == 0) s_cflag[(k + 2) % 3] = 0;
    }
    if (own && p * kPage < nw && p < pc1) {  // (the loop runs past pc1 to a multiple of kDepth)
      // the four 16-entry groups of the page; one reduce-scatter across the
      // lane rows then leaves the 64-head sum of group r in row r, so each
      // lane holds one logit and the wave stores the page's 64 logits at once
      float pk[kPage / 16];
#pragma unroll
      for (int g = 0; g < kPage / 16; ++g) {
        pk[g] = 0.f;
        if (g % kWpr != sub) continue;  // another wave of the row scores group g
        const int e = g * 16 + col;
        v8i bb;
        int sb = 127;
        if (kFp4) {
          const int pos = grp ^ ((e >> 2) & 3);
          const v4i x = *reinterpret_cast<const v4i*>(&s_b[buf][e * kRowBytes + pos * 16]);
          bb = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
          sb = (s_bs[buf][e] >> (8 * grp)) & 0xFF;
        } else {
          const v4i x = *reinterpret_cast<const v4i*>(&s_b[buf][e * kRowBytes + ((2 * grp) ^ (e & 7)) * 16]);
          const v4i y = *reinterpret_cast<const v4i*>(&s_b[buf][e * kRowBytes + ((2 * grp + 1) ^ (e & 7)) * 16]);
          bb = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        }
        pk[g] = head_sum(bb, sb);
      }
      const float tot = rows4_reduce_scatter(pk[0], pk[1], pk[2], pk[3]);
      const int e = grp * 16 + col;  // the entry whose logit this lane holds
      const float ks = kFp4 ? 1.f : __uint_as_float(s_bs[buf][e]);
      if constexpr (kSel) {
        const int j = p * kPage + e;
        if (cflag && sel.cnt > kTopK) sel.compact(false);
        sel.push(tot * ks, (uint32_t)(j - jbase), j < nw);
        if (lane == 0 && sel.short_of_room()) s_cflag[(k + 1) % 3] = 1;
      } else {
        const int off = grp % kWpr == sub ? (p * kPage + e) * 4 : 0x7FFFFFFF;  // past the buffer: dropped
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot * ks), out_rsrc, off, 0, 0);
      }
    }
  };
  static_assert(kDepth == 3, "the page loop below is unrolled by hand for three slots");
  // steps past the last page only stage (clamped) and synchronise: no branch
  // inside the loop keeps the load counters exact across its back edge
  for (int p0 = pc0; p0 < npages; p0 += kDepth) {
    page_step(p0, std::integral_constant<int, 0>{});
    page_step(p0 + 1, std::integral_constant<int, 1>{});
    page_step(p0 + 2, std::integral_constant<int, 2>{});
  }
  // a row of another sequence: its own pages of the range, read straight from
  // memory (the row's waves take turns by 16-entry group)
  if (!own && row_ok) {
    const int jend = min(nw, pc1 * kPage);
    for (int j0 = pc0 * kPage + 16 * sub; j0 < jend; j0 += 16 * kWpr) {
      const int e = j0 + col;
      const int ee = min(e, nw - 1);
      const int64_t slot = (int64_t)ptw[ee / kPage] * kPage + ee % kPage;
      const uint8_t* q = kdata + slot * kRowBytes + grp * (kRowBytes / 4);
      const v4i x = *reinterpret_cast<const v4i*>(q);
      v8i bb;
      int sb = 127;
      float ks = 1.f;
      if (kFp4) {
        bb = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        sb = reinterpret_cast<const uint8_t*>(kscale)[slot * 4 + grp];
      } else {
        const v4i y = *reinterpret_cast<const v4i*>(q + 16);
        bb = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        ks = reinterpret_cast<const float*>(kscale)[slot];
      }
      score_store(bb, sb, ks, e);
    }
  }
  if constexpr (kSel) {
    if (!row_ok) return;
    sel.finish();
    const int32_t* ptr = pt + (int64_t)seqw * pt_stride;
    const bool direct = gridDim.y == 1;  // one range: the row's selection itself
    const int64_t o = ((int64_t)t * gridDim.y + blockIdx.y) * kTopK;
    for (int q = lane; q < kTopK; q += 64) {
      const bool have = q < sel.cnt;
      const int32_t j = have ? jbase + (int32_t)sel.idx[q] : -1;
      const int32_t phys = have ? (int32_t)((int64_t)ptr[j / kPage] * kPage + j % kPage) : -1;
      if (direct) {
        co.phys_idx[o + q] = phys;
        if (co.logical_idx) co.logical_idx[o + q] = j;
      } else {
        co.keys[o + q] = have ? sel.key[q] : 0u;
        co.js[o + q] = have ? j : INT_MAX;
        co.phys[o + q] = phys;
      }
    }
  }
}

// fp32 path (small indexers: H_I * D_I <= 8192, D_I in {64, 128}). A wave
// scores 16 consecutive entries: lane (e, part) = (lane / 4, lane % 4) holds a
// quarter of entry e's row in registers (the wave reads 16 rows of a page as
// coalesced 16-byte loads), the query and head weights sit in LDS (read as
// broadcasts), and each head's dot product is finished across the four lanes
// of a quad by two DPP moves.
template <int kD>
__global__ void __launch_bounds__(256)
indexer_f32_kernel(const float* __restrict__ q, const float* __restrict__ w, int H,
                   const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_len,
                   const int32_t* __restrict__ pt, int pt_stride,
                   const float* __restrict__ kdata, int page_size, float* __restrict__ logits,
                   int64_t ld) {
  constexpr int kQ = kD / 4;  // floats of a row per lane
  extern __shared__ __attribute__((aligned(16))) float sq[];  // [H][kD] then w[H]
  const int t = blockIdx.y;
  for (int i = threadIdx.x; i < H * kD / 4; i += blockDim.x)
    reinterpret_cast<float4*>(sq)[i] = reinterpret_cast<const float4*>(q + (int64_t)t * H * kD)[i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) sq[H * kD + i] = w[(int64_t)t * H + i];
  __syncthreads();
  const int n = row_len[t];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = lane >> 2, part = lane & 3;
  const int jw = blockIdx.x * 64 + wave * 16;  // first entry of this wave
  if (jw >= n) return;                          // wave-uniform; no barrier follows
  const int j = jw + e;
  const int jj = min(j, n - 1);
  const int64_t slot =
      (int64_t)pt[(int64_t)row_seq[t] * pt_stride + jj / page_size] * page_size + jj % page_size;
  float k[kQ];
#pragma unroll
  for (int i = 0; i < kQ; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(kdata + slot * kD + part * kQ + i);
    k[i] = v.x;
    k[i + 1] = v.y;
    k[i + 2] = v.z;
    k[i + 3] = v.w;
  }
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    const float* qh = sq + h * kD + part * kQ;
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < kQ; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(qh + i);
      d = fmaf(a.x, k[i], fmaf(a.y, k[i + 1], fmaf(a.z, k[i + 2], fmaf(a.w, k[i + 3], d))));
    }
    d += lane_xor<1>(d);
    d += lane_xor<2>(d);
    acc = fmaf(sq[H * kD + h], fmaxf(d, 0.f), acc);
  }
  if (part == 0 && j < n) logits[(int64_t)t * ld + j] = acc;
}

}  // namespace

size_t indexer_ws_bytes(int64_t T, int H_I) {
  // prepared query codes (<= 128 B per head) + scales (<= 4 B per head), 256-B aligned
  const size_t codes = ((size_t)T * H_I * kDim + 255) & ~(size_t)255;
  return codes + (((size_t)T * H_I * 4 + 255) & ~(size_t)255);
}

// Entries per scan workgroup: the rows are chunked so the grid has ~256
// workgroups (one per CU), each wave a long stream: measured on MI355X, one
// workgroup per CU streams faster than two (fewer concurrent page streams).
static int64_t scan_chunk(int64_t T, int64_t max_row_len) {
  const int64_t target = kScanSlots;
  const int64_t total = T * max_row_len;
  int64_t chunk = total / target;
  chunk = ((chunk + kWgEntries - 1) / kWgEntries) * kWgEntries;
  if (chunk < kWgEntries) chunk = kWgEntries;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  return chunk;
}

// Rows per workgroup of the row-block kernel for this call, or 0 for the
// per-row scan. Rows that come in groups sharing a sequence (the prep flags'
// rows-per-sequence hint g >= 2) take it with the largest divisor of g in
// 2..8 (none: a prime above 8); otherwise many rows (prefill) take it with 8.
// Only 64-entry pages.
static int rows_kernel_rows(int64_t T, const csa_index_pool& k, uint32_t prep) {
  if (k.page_size != 64) return 0;
  const int g = (int)((prep >> 8) & 0xFFu);
  if (g >= 2) {
    for (int r = kRowsPerWG; r >= 2; --r)
      if (g % r == 0) return r;
    return 0;
  }
  return T >= kRowsPerWG * 32 ? 8 : 0;
}

// Page ranges of the row-block kernel (blockIdx.y) and pages per range: about
// two workgroups per CU when the row groups are few (measured for 32 sequences
// x 4 rows at 128K: 58 us with 256 workgroups, 47 with 512, 51 with 1024). The
// fused selection takes at least 8 pages (512 entries) per range, so that only
// a row's last ranges write padding candidates, after all its entries, at most
// kCandFinalMax / 512 ranges, the final pass's capacity, and at most kSelSpan
// entries per range (its buffer holds 16-bit entry offsets); rows beyond
// kCandFinalMax / 512 * kSelSpan entries do not take it.
static int rows_ranges(int64_t T, int rows, int64_t max_row_len, bool sel, int& ppc) {
  const int64_t groups = (T + rows - 1) / rows;
  const int64_t pages = (max_row_len + 63) / 64;
  int64_t ranges = std::max<int64_t>(1, std::min<int64_t>(pages, (512 + groups - 1) / groups));
  if (sel) {
    const int64_t span = (pages * 64 + kSelSpan - 1) / kSelSpan;  // 16-bit offsets within a range
    ranges = std::max<int64_t>(span, std::min<int64_t>({ranges, pages / 8, kCandFinalMax / kTopK}));
  }
  ppc = (int)((pages + ranges - 1) / ranges);
  return (int)((pages + ppc - 1) / ppc);
}

int indexer_rows_sel_ranges(int64_t T, int H_I, int D_I, const csa_index_pool& k,
                            int64_t max_row_len, uint32_t prep) {
  if (k.fmt != CSA_FP8_E4M3 && k.fmt != CSA_MXFP4) return 0;
  if (H_I != kHeads || D_I != kDim || T == 0 || max_row_len == 0) return 0;
  const int rows = rows_kernel_rows(T, k, prep);
  // 8 rows only: with fewer, one wave per row (the selection's unit) leaves
  // waves idle (multi-token decode, 4 rows: 77.8 us vs 49.5 + 20.0 us of
  // logits and two-pass top-512)
  if (rows != kRowsPerWG) return 0;
  int ppc;
  const int ranges = rows_ranges(T, rows, max_row_len, true, ppc);
  return ranges * kTopK <= kCandFinalMax ? ranges : 0;
}

int64_t indexer_rows_sel_cands(int64_t T, int64_t max_row_len) {
  if (T == 0 || max_row_len == 0) return 0;
  int ppc;
  const int ranges = rows_ranges(T, kRowsPerWG, max_row_len, true, ppc);
  return ranges > 1 && ranges * kTopK <= kCandFinalMax ? (int64_t)ranges * kTopK : 0;
}

int64_t indexer_scan_chunks(int64_t T, int64_t max_row_len) {
  const int64_t c = scan_chunk(T, max_row_len);
  return (max_row_len + c - 1) / c;
}

int indexer_cand_chunks(int64_t T, int H_I, int D_I, const csa_index_pool& k,
                        int64_t max_row_len, uint32_t prep) {
  if (k.fmt != CSA_FP8_E4M3 && k.fmt != CSA_MXFP4) return 0;
  if (H_I != kHeads || D_I != kDim || k.page_size % 16 != 0) return 0;
  if (T == 0 || max_row_len == 0 || rows_kernel_rows(T, k, prep)) return 0;
  const int64_t chunks = indexer_scan_chunks(T, max_row_len);
  return chunks * kTopK <= (int64_t)kCandGroups * kCandFinalMax ? (int)chunks : 0;
}

hipError_t launch_indexer(const void* q, int q_fmt, const void* q_scale, uint32_t prep,
                          const float* w, int T, int H_I, int D_I, const int32_t* row_seq,
                          const int32_t* row_len, int max_row_len, const int32_t* page_table,
                          int pt_stride, const csa_index_pool& k, float* logits, int64_t ld,
                          void* q_used, void* q_used_scale, void* ws, hipStream_t s,
                          const CandOut* cand) {
  if (T == 0 || max_row_len == 0) return hipSuccess;
  if (k.fmt == CSA_F32) {
    dim3 grid((max_row_len + 63) / 64, T);
    const size_t lds = ((size_t)H_I * D_I + H_I) * sizeof(float);
    if (D_I == 64)
      hipLaunchKernelGGL(indexer_f32_kernel<64>, grid, dim3(256), lds, s, (const float*)q, w, H_I,
                         row_seq, row_len, page_table, pt_stride, (const float*)k.data, k.page_size,
                         logits, ld);
    else
      hipLaunchKernelGGL(indexer_f32_kernel<128>, grid, dim3(256), lds, s, (const float*)q, w, H_I,
                         row_seq, row_len, page_table, pt_stride, (const float*)k.data, k.page_size,
                         logits, ld);
    return hipGetLastError();
  }
  const uint8_t* qc = (const uint8_t*)q;
  const void* qs = q_scale;
  if (prep & CSA_PREP_QUANT) {
    // Prepare the query rows once (rotation + quantisation) into q_used or the
    // workspace, then score from the prepared codes.
    void* dst = q_used;
    void* dsts = q_used_scale;
    if (!dst) {
      dst = ws;
      dsts = (uint8_t*)ws + (((size_t)T * H_I * kDim + 255) & ~(size_t)255);
    }
    const csa_rope no_rope{nullptr, nullptr, 0, 1};
    hipError_t e = launch_index_prep(q, q_fmt, (int64_t)T * H_I, D_I,
                                     prep & (CSA_PREP_HADAMARD | CSA_PREP_QUANT), k.fmt, dst, dsts,
                                     nullptr, no_rope, s);
    if (e != hipSuccess) return e;
    qc = (const uint8_t*)dst;
    qs = dsts;
  } else if (q_used) {
    const size_t code_bytes = (size_t)T * H_I * (k.fmt == CSA_MXFP4 ? kDim / 2 : kDim);
    const size_t scale_bytes = (size_t)T * H_I * 4;
    hipError_t e = hipMemcpyAsync(q_used, q, code_bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(q_used_scale, q_scale, scale_bytes, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
  const int64_t chunk = scan_chunk(T, max_row_len);
  const bool rsel = cand && cand->rows_sel;
  const int rows = (rsel || !cand) ? rows_kernel_rows(T, k, prep) : 0;
  if (rows) {
    const int groups = (int)((T + rows - 1) / rows);
    int ppc;
    const int ranges = rows_ranges(T, rows, max_row_len, rsel, ppc);
    dim3 g2(groups, ranges);
    const CandOut co = rsel ? *cand : CandOut{};
#define CSA_ROWS(FP4, R, SEL)                                                                     \
  hipLaunchKernelGGL((indexer_rows_kernel<FP4, R, SEL>), g2, dim3(kRowsPerWG * 64), 0, s, qc, qs, \
                     w, row_seq, row_len, T, page_table, pt_stride, (const uint8_t*)k.data,       \
                     k.scale, logits, ld, ppc, co)
    const bool fp4 = k.fmt == CSA_MXFP4;
    if (rsel) {  // rows == 8 (indexer_rows_sel_ranges)
      if (fp4) CSA_ROWS(true, kRowsPerWG, true);
      else CSA_ROWS(false, kRowsPerWG, true);
      return hipGetLastError();
    }
#define CSA_ROWS_CASE(R)                        \
  case R:                                       \
    if (fp4) CSA_ROWS(true, R, false);          \
    else CSA_ROWS(false, R, false);             \
    break;
    switch (rows) {
      CSA_ROWS_CASE(2)
      CSA_ROWS_CASE(3)
      CSA_ROWS_CASE(4)
      CSA_ROWS_CASE(5)
      CSA_ROWS_CASE(6)
      CSA_ROWS_CASE(7)
      default: CSA_ROWS_CASE(8)
    }
#undef CSA_ROWS_CASE
#undef CSA_ROWS
    return hipGetLastError();
  }
  // The grid covers the rows in 4096-entry chunks. A long ragged batch (more
  // entries than kScanSlots such chunks) takes indexer_wide_kernel over as
  // many workgroups, one per work item of the plan wide_item makes on the
  // device (the candidate slots stay those of 4096-entry chunks).
  dim3 grid((unsigned)((max_row_len + chunk - 1) / chunk), T);
  CandOut co = cand ? *cand : CandOut{};
  const bool wide = cand && k.page_size == 64 && T <= kWideRows &&
                    (int64_t)T * max_row_len > (int64_t)kScanSlots * kMaxChunk;
  if (wide) {
    co.wide_rows = T;
    co.wide_chunks = (int)grid.x;
    const dim3 g1(grid.x * grid.y);
#define CSA_WIDE(FP4)                                                                             \
  hipLaunchKernelGGL((indexer_wide_kernel<FP4>), g1, dim3(idx_threads<true>()), 0, s, qc, qs, w, \
                     row_seq, row_len, page_table, pt_stride, (const uint8_t*)k.data, k.scale, co)
    if (k.fmt == CSA_MXFP4) CSA_WIDE(true);
    else CSA_WIDE(false);
#undef CSA_WIDE
    return hipGetLastError();
  }
#define CSA_IDX(FP4, P64, CAND)                                                                    \
  hipLaunchKernelGGL((indexer_mfma_kernel<FP4, P64, CAND>), grid, dim3(idx_threads<CAND>()), 0, s, qc, qs, \
                     w, row_seq, row_len, page_table, pt_stride, (const uint8_t*)k.data, k.scale,  \
                     k.page_size, logits, ld, (int)chunk, co)
#define CSA_IDX_P(FP4, CAND)                 \
  if (k.page_size == 64) CSA_IDX(FP4, true, CAND); \
  else CSA_IDX(FP4, false, CAND);
  if (cand) {
    if (k.fmt == CSA_MXFP4) { CSA_IDX_P(true, true) }
    else { CSA_IDX_P(false, true) }
  } else {
    if (k.fmt == CSA_MXFP4) { CSA_IDX_P(true, false) }
    else { CSA_IDX_P(false, false) }
  }
#undef CSA_IDX_P
#undef CSA_IDX
  return hipGetLastError();
}

}  // namespace csa
