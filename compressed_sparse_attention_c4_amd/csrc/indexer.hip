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

namespace csa {
namespace {

constexpr int kHeads = 64;   // indexer heads handled by the MFMA path
constexpr int kDim = 128;    // indexer head dim handled by the MFMA path
constexpr int kWaves = 4;
constexpr int kRing = 2;     // 64-entry batches in flight per wave
constexpr int kWgEntries = kWaves * kRing * 64;
constexpr int kMaxChunk = 8 * kWgEntries;  // entries per workgroup, at most

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
// kWaves scan, all of them select (fewer keys per lane, the same barriers).
constexpr int kSelWaves = 8;
template <bool kCand>
constexpr int idx_threads() { return (kCand ? kSelWaves : kWaves) * 64; }

template <bool kFp4, bool kPage64, bool kCand>
__global__ void __launch_bounds__(idx_threads<kCand>())
indexer_mfma_kernel(const uint8_t* __restrict__ qc, const void* __restrict__ qs,
                    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ row_len, const int32_t* __restrict__ pt,
                    int pt_stride, const uint8_t* __restrict__ kdata,
                    const void* __restrict__ kscale, int page_size, float* __restrict__ logits,
                    int64_t ld, int chunk, uint32_t* __restrict__ okeys,
                    int32_t* __restrict__ ojs, int32_t* __restrict__ ophys) {
  constexpr int kRowBytes = kFp4 ? kDim / 2 : kDim;  // bytes per index-K / q row
  __shared__ int32_t s_pages[kMaxChunk / 16 + 2];      // physical pages of this chunk
  __shared__ __attribute__((aligned(16))) float s_out[kMaxChunk + 64];  // the chunk's logits
  const int t = blockIdx.y;
  const int n = row_len[t];
  const int c0 = blockIdx.x * chunk;
  if (c0 >= n) {
    if constexpr (kCand) {
      for (int p = threadIdx.x; p < kTopK; p += idx_threads<kCand>()) {
        const int64_t o = ((int64_t)t * gridDim.x + blockIdx.x) * kTopK + p;
        okeys[o] = 0u;
        ojs[o] = INT_MAX;
        ophys[o] = -1;
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

  if (kCand && wave >= kWaves) {
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
  // w + kWaves, ... and keeps kRing batches of loads in flight (a register
  // ring, slot = batch % kRing). After the 16 MFMAs of a batch, one
  // reduce-scatter across the four lane rows leaves in row r the 64-head sum
  // of group r, so each lane stores one logit and a wave writes the batch's
  // 64 logits as one contiguous 256-byte store; the lane also loads the FP8
  // scale of exactly that entry. The logits collect in LDS and are written
  // out after the loop: a global store inside it would sit in the same
  // in-order memory counter as the loads and delay every later wait. The loop
  // is branch-free: batches past the chunk load entry 0 of its first page (or
  // their page), and their logits land in LDS past the chunk and are dropped.
  const int nbatch = (c1 - c0 + 63) / 64;
  const int nb = (nbatch - wave + kWaves - 1) / kWaves;  // batches of this wave
  v8i b[kRing][4];
  int sb[kRing][4];
  float ks[kRing];
  auto slot_of = [&](int j, int g0) __attribute__((always_inline)) {
    const int pg = s_pages[g0 < c1 ? g0 / page_size - pg0 : 0];
    return (j < c1) ? (int64_t)pg * page_size + j % page_size : (int64_t)s_pages[0] * page_size;
  };
  // 64-entry pages (the C4 layout): a batch is one page (the chunk starts on a
  // page), found with no division; entries past the chunk read their page
  // anyway (their logits are dropped)
  const int last_pg = npg - 1;
  auto batch_page = [&](int i) __attribute__((always_inline)) {
    return (int64_t)s_pages[min(i * kWaves + wave, last_pg)] * 64;
  };
  auto issue = [&](int i, auto R) __attribute__((always_inline)) {
    constexpr int r = decltype(R)::value;
    const int e0 = c0 + (i * kWaves + wave) * 64;  // first entry of the batch
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
  auto step = [&](int i, auto R) __attribute__((always_inline)) {
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
    const int jl = i < nb ? (i * kWaves + wave) * 64 + 16 * grp + col : kMaxChunk + lane;
    s_out[jl] = tot * ks[r];
    issue(i + kRing, R);  // refill the slot just consumed
  };
  static_assert(kRing == 2, "the batch loop below is unrolled by hand for two slots");
  issue(0, std::integral_constant<int, 0>{});
  issue(1, std::integral_constant<int, 1>{});
  for (int i0 = 0; i0 < nb; i0 += kRing) {
    step(i0, std::integral_constant<int, 0>{});
    step(i0 + 1, std::integral_constant<int, 1>{});
  }
  }  // scan waves
  __syncthreads();
  const int n_out = c1 - c0;
  if constexpr (kCand) {
    // keys from LDS: element seg + 64 i + lane of this wave's segment
    constexpr int kTH = idx_threads<kCand>();
    constexpr int kE = kMaxChunk / kTH;
    __shared__ TopkLds L;
    for (int i = threadIdx.x; i < kTopkBins; i += kTH) L.hist[i] = 0u;
    const int seg = wave * 64 * kE;
    uint32_t kr[kE];
#pragma unroll
    for (int i = 0; i < kE; ++i) {
      const int e = seg + 64 * i + lane;
      kr[i] = e < n_out ? float_key(s_out[e]) : 0u;
    }
    const int K = min(kTopK, n_out);
    topk_select<kE, kTH>(kr, n_out, K, seg, L);
    for (int p = threadIdx.x; p < kTopK; p += kTH) {
      const int64_t o = ((int64_t)t * gridDim.x + blockIdx.x) * kTopK + p;
      uint32_t key = 0u;  // padding past K
      int32_t j = INT_MAX, phys = -1;
      if (p < K) {
        key = L.out_k[p];
        j = c0 + L.out_e[p];
        phys = s_pages[j / page_size - pg0] * page_size + j % page_size;  // a page of this chunk
      }
      okeys[o] = key;
      ojs[o] = j;
      ophys[o] = phys;
    }
  } else {
    float* orow = logits + (int64_t)t * ld + c0;
    for (int j = threadIdx.x; j < n_out; j += kWaves * 64) orow[j] = s_out[j];
  }
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
constexpr int kRowsPerWG = 8;  // waves per workgroup (and rows, at most)

template <bool kFp4, int kRows>
__global__ void __launch_bounds__(kRowsPerWG * 64)
indexer_rows_kernel(const uint8_t* __restrict__ qc, const void* __restrict__ qs,
                    const float* __restrict__ w, const int32_t* __restrict__ row_seq,
                    const int32_t* __restrict__ row_len, int T, const int32_t* __restrict__ pt,
                    int pt_stride, const uint8_t* __restrict__ kdata,
                    const void* __restrict__ kscale, float* __restrict__ logits, int64_t ld,
                    int ppc) {
  static_assert(kRows >= 2 && kRows <= kRowsPerWG, "rows per workgroup");
  constexpr int kWpr = kRowsPerWG / kRows;  // waves per row
  constexpr int kPage = 64;                          // entries per page (= tile)
  constexpr int kRowBytes = kFp4 ? kDim / 2 : kDim;  // bytes per index-K row
  constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kPage * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s_bs[2][kPage];  // fp32 scale / 4 e8m0 bytes
  __shared__ int s_len[kRows];

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
  const int npages = min((maxall + kPage - 1) / kPage, pc1);
  const int nstage = min((maxown + kPage - 1) / kPage, pc1);
  const __amdgpu_buffer_rsrc_t out_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(logits + (int64_t)tq * ld, (short)0, nw * 4, 0x00020000);
  const int32_t* pt0 = pt + (int64_t)seq0 * pt_stride;
  const int32_t* ptw = pt + (int64_t)seqw * pt_stride;

  // staging: thread i < kPage*kChunks moves chunk (i % kChunks) of entry i / kChunks.
  // Every thread issues the loads (spare threads duplicate a chunk) so that
  // the loop holds no conditional load and outstanding loads stay countable.
  const bool stager = tid < kPage * kChunks;
  const int stid = tid % (kPage * kChunks);
  const int se = stid / kChunks, sc = stid % kChunks;
  const int sw = kFp4 ? (sc ^ ((se >> 2) & 3)) : (sc ^ (se & 7));  // swizzled chunk position
  const bool scaler = tid < kPage / 4;  // 16 threads also move the page's 256 B of scales
  const int sce = (tid % (kPage / 4)) * 4;  // first of 4 entries whose scales this thread moves
  // pages are loaded kDepth pages ahead into a register ring (slot p % kDepth)
  constexpr int kDepth = 3;
  v4i stage[kDepth], sstage[kDepth];  // native vectors (HIP's uint4 struct blocks promotion)
  auto load_page = [&](int p, auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    // clamped, never skipped; with no page to stage, pool page 0 stands in
    const int64_t base = nstage > 0 ? (int64_t)pt0[min(p, nstage - 1)] * kPage : 0;
    stage[k] = *reinterpret_cast<const v4i*>(kdata + (base + se) * kRowBytes + sc * 16);
    sstage[k] = *reinterpret_cast<const v4i*>(reinterpret_cast<const uint8_t*>(kscale) + (base + sce) * 4);
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
  auto head_sum = [&](const v8i& bb, int sb) __attribute__((always_inline)) {
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
    const int off = grp == 0 ? jrow * 4 : 0x7FFFFFFF;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v * ks), out_rsrc, off, 0, 0);
  };
  auto page_step = [&](const int p, auto K) __attribute__((always_inline)) {
    constexpr int k = decltype(K)::value;
    const int buf = p & 1;
    if (stager) *reinterpret_cast<v4i*>(&s_b[buf][se * kRowBytes + sw * 16]) = stage[k];
    if (scaler) *reinterpret_cast<v4i*>(&s_bs[buf][sce]) = sstage[k];
    __syncthreads();
    load_page(p + kDepth, K);  // refill the slot just written to LDS
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
      const int off = grp % kWpr == sub ? (p * kPage + e) * 4 : 0x7FFFFFFF;  // past the buffer: dropped
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tot * ks), out_rsrc, off, 0, 0);
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
}

// fp32 path (small indexers, any H_I, D_I in {64, 128}): one thread per entry,
// the row's query in LDS.
__global__ void __launch_bounds__(256)
indexer_f32_kernel(const float* __restrict__ q, const float* __restrict__ w, int H, int D,
                   const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_len,
                   const int32_t* __restrict__ pt, int pt_stride,
                   const float* __restrict__ kdata, int page_size, float* __restrict__ logits,
                   int64_t ld) {
  extern __shared__ float sq[];  // [H][D] then w[H]
  const int t = blockIdx.y;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) sq[i] = q[(int64_t)t * H * D + i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) sq[H * D + i] = w[(int64_t)t * H + i];
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= row_len[t]) return;
  const int64_t slot = (int64_t)pt[(int64_t)row_seq[t] * pt_stride + j / page_size] * page_size + j % page_size;
  const float* k = kdata + slot * D;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    float d = 0.f;
    for (int i = 0; i < D; i += 4) {
      float4 kv = *reinterpret_cast<const float4*>(k + i);
      d = fmaf(sq[h * D + i], kv.x, d);
      d = fmaf(sq[h * D + i + 1], kv.y, d);
      d = fmaf(sq[h * D + i + 2], kv.z, d);
      d = fmaf(sq[h * D + i + 3], kv.w, d);
    }
    acc = fmaf(sq[H * D + h], fmaxf(d, 0.f), acc);
  }
  logits[(int64_t)t * ld + j] = acc;
}

}  // namespace

size_t indexer_ws_bytes(int64_t T, int H_I) {
  // prepared query codes (<= 128 B per head) + scales (<= 4 B per head), 256-B aligned
  const size_t codes = ((size_t)T * H_I * kDim + 255) & ~(size_t)255;
  return codes + (((size_t)T * H_I * 4 + 255) & ~(size_t)255);
}

// Entries per scan workgroup: the rows are chunked so the grid has ~256
// workgroups (one per CU), each wave a long stream: measured on MI355X, one
// workgroup per CU streams faster than two (fewer concurrent page streams);
// CSA_TUNE_INDEXER_WGS overrides the target (tuning only).
static int64_t scan_chunk(int64_t T, int64_t max_row_len) {
  int64_t target = 256;
  if (const char* e = getenv("CSA_TUNE_INDEXER_WGS")) target = atoll(e) > 0 ? atoll(e) : target;
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
  if (k.page_size != 64 || getenv("CSA_TUNE_INDEXER_NO_ROWS")) return 0;
  const int g = (int)((prep >> 8) & 0xFFu);
  if (g >= 2) {
    for (int r = kRowsPerWG; r >= 2; --r)
      if (g % r == 0) return r;
    return 0;
  }
  return T >= kRowsPerWG * 32 ? 8 : 0;
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
                          uint32_t* okeys, int32_t* ojs, int32_t* ophys) {
  if (T == 0 || max_row_len == 0) return hipSuccess;
  if (k.fmt == CSA_F32) {
    dim3 grid((max_row_len + 255) / 256, T);
    const size_t lds = ((size_t)H_I * D_I + H_I) * sizeof(float);
    hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), lds, s, (const float*)q, w, H_I,
                       D_I, row_seq, row_len, page_table, pt_stride, (const float*)k.data,
                       k.page_size, logits, ld);
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
    hipError_t e = launch_index_prep(q, q_fmt, (int64_t)T * H_I, D_I,
                                     prep & (CSA_PREP_HADAMARD | CSA_PREP_QUANT), k.fmt, dst, dsts,
                                     nullptr, s);
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
  const int rows = okeys ? 0 : rows_kernel_rows(T, k, prep);
  if (rows) {
    // page ranges: about two workgroups per CU when the row groups are few
    // (measured for 32 sequences x 4 rows at 128K: 58 us with 256 workgroups,
    // 47 with 512, 51 with 1024)
    const int groups = (int)((T + rows - 1) / rows);
    const int pages = (int)((max_row_len + 63) / 64);
    const int ranges = std::max(1, std::min(pages, (512 + groups - 1) / groups));
    const int ppc = (pages + ranges - 1) / ranges;
    dim3 g2(groups, (pages + ppc - 1) / ppc);
#define CSA_ROWS(FP4, R)                                                                          \
  hipLaunchKernelGGL((indexer_rows_kernel<FP4, R>), g2, dim3(kRowsPerWG * 64), 0, s, qc, qs, w,   \
                     row_seq, row_len, T, page_table, pt_stride, (const uint8_t*)k.data, k.scale, \
                     logits, ld, ppc)
    const bool fp4 = k.fmt == CSA_MXFP4;
#define CSA_ROWS_CASE(R)                        \
  case R:                                       \
    if (fp4) CSA_ROWS(true, R);                 \
    else CSA_ROWS(false, R);                    \
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
  dim3 grid((unsigned)((max_row_len + chunk - 1) / chunk), T);
#define CSA_IDX(FP4, P64, CAND)                                                                    \
  hipLaunchKernelGGL((indexer_mfma_kernel<FP4, P64, CAND>), grid, dim3(idx_threads<CAND>()), 0, s, qc, qs, \
                     w, row_seq, row_len, page_table, pt_stride, (const uint8_t*)k.data, k.scale,  \
                     k.page_size, logits, ld, (int)chunk, okeys, ojs, ophys)
#define CSA_IDX_P(FP4, CAND)                 \
  if (k.page_size == 64) CSA_IDX(FP4, true, CAND); \
  else CSA_IDX(FP4, false, CAND);
  if (okeys) {
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
