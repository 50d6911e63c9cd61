// wave_topk.hpp -- one wavefront's running top-K over a row whose elements
// arrive in increasing index order ("Token 的一生：DSV4 架构与 DSpark" §3.2: the
// top-512 of each query row's indexer logits), so that a kernel that produces
// the logits can select from them without writing them out.
//
// Order, as the top-512 kernel's: larger key first, equal keys by lower index.
// Keys are the order-preserving uint32 image of the logit (key 0: NaN).
//
// The wave keeps a buffer of candidates (key, index - base as 16 bits) in LDS,
// in arrival order, and a threshold `thr` that never exceeds the K-th largest
// key seen so far. Elements arrive with a cheaper pre-key (the sign-flip image
// of the float's bits: equal to the key except that -0 sits one below +0 and
// NaNs fall outside the keys of -inf..+inf); the buffer's pre-keys are turned
// into keys when it is compacted and when it is finished, and thr is never
// the one value (that of -0) where comparing a pre-key and comparing the key
// against it could differ. An element whose key is not above thr is dropped as it
// arrives: at least K elements seen before it have a key >= thr >= its key and
// a lower index, so all of them rank above it. When the buffer runs short of
// room it is compacted. A histogram of the buffer's keys (this wave alone; 256
// LDS bins over the buffer's key range, so keys that crowd into a narrow
// range still spread out) gives the bin holding the K-th largest key:
//   - approximate (while scanning): every element from that bin's lower edge
//     up is kept, in order, and the edge becomes the threshold (it is <= the
//     K-th largest key); taken when that frees enough room;
//   - exact (at the end, or when the bin is too full): the bins are refined
//     over the lower bits (radix select) to the K-th largest key t and the
//     number `need` of keys equal to t within the top K; the buffer keeps its
//     elements with key > t and the first `need` with key == t: its top K.
// After the final exact compaction the buffer holds the row's top K in
// increasing index order, the order in which the top-512 kernel emits them.
//
// The buffer and histogram belong to this wave only: no workgroup barrier is
// used. A wavefront executes its LDS instructions in order, so the wave's own
// reads see its earlier writes; wave_barrier() keeps the compiler from moving
// LDS accesses across the phases.
#pragma once
#include "csa_device.hpp"

namespace csa {

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int kCap, int kK>
struct WaveTopk {
  static_assert(kCap % 64 == 0 && kCap >= kK + 256, "buffer holds K plus a few batches");
  static constexpr int kPer = kCap / 64;  // buffer elements per lane at compaction
  static constexpr int kRoom = 192;       // room an approximate compaction must leave
  uint32_t* key;   // LDS [kCap]
  uint16_t* idx;   // LDS [kCap]: index - base
  uint32_t* hist;  // LDS [256]
  int cnt = 0;     // elements in the buffer (wave-uniform)
  int nkey = 0;    // elements [0, nkey) hold keys, the later ones pre-keys
  uint32_t thr = 0u;
  bool thr_set = false;  // before the first compaction every element is taken

  // Offers this lane's element (logit v, index base + j16) when valid. Every
  // lane of the wave calls it; the indices offered over the calls increase.
  // Compacts when the buffer could not take the next 64 elements.
  __device__ __forceinline__ void push(float v, uint32_t j16, bool valid) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // pre-key
    const bool acc = valid && (!thr_set || k > thr);
    const uint64_t m = __ballot(acc);
    if (acc) {
      const int pos = cnt + (int)lanes_below(m);
      key[pos] = k;
      idx[pos] = (uint16_t)j16;
    }
    cnt += __popcll(m);
    if (cnt > kCap - 64) compact(false);
  }

  // True when the buffer may not take two more 64-element batches.
  __device__ __forceinline__ bool short_of_room() const { return cnt > kCap - 128; }

  // The key of a pre-key: -0 ranks as +0, NaN as 0.
  static __device__ __forceinline__ uint32_t key_of(uint32_t pk) {
    return pk == 0x7FFFFFFFu ? 0x80000000u : (pk > 0xFF800000u || pk < 0x007FFFFFu ? 0u : pk);
  }

  // Reduces the buffer to its exact top K (when it holds more), in order, and
  // leaves keys (not pre-keys) in all of it.
  __device__ __forceinline__ void finish() {
    if (cnt > kK) {
      compact(true);
      return;
    }
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_wave_barrier();
    for (int e = nkey + lane; e < cnt; e += 64) key[e] = key_of(key[e]);
    __builtin_amdgcn_wave_barrier();
    nkey = cnt;
  }

  __device__ __forceinline__ void compact(bool exact) {
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_wave_barrier();
    // the keys are read from LDS in every pass (held in registers they would
    // add to the pressure of the loop around the call)
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll 2
    for (int i = 0; i < kPer; ++i) {
      const int e = i * 64 + lane;
      uint32_t kv = key[e];
      if (e >= nkey && e < cnt) {  // pre-key -> key
        kv = key_of(kv);
        key[e] = kv;
      }
      if (e < cnt) {
        lo = min(lo, kv);
        hi = max(hi, kv);
      }
    }
    lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_umin(lo));
    hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)wave_umax(hi));
    // ---- radix select of the K-th largest key: d = key - lo, fixed from the top
    const uint32_t range = hi - lo;
    int s = range == 0u ? 0 : max(0, (32 - __clz(range)) - 8);  // shift of this pass's digit
    int sp = 32;          // shift of the part fixed so far (32: nothing fixed)
    uint32_t fixed = 0u;  // d >> sp of the keys still in the race
    uint32_t k = kK;      // rank sought among them
    bool approx = false;  // keep every key >= edge instead of the exact top K
    uint32_t edge = 0u;
    while (true) {
      __builtin_amdgcn_wave_barrier();
      reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
      __builtin_amdgcn_wave_barrier();
      // the digit: bits [s, sp) of d (the first pass: d >> s < 256 by the choice of s)
      const uint32_t dmask = sp >= 32 ? 255u : (1u << (sp - s)) - 1u;
#pragma unroll 2
      for (int i = 0; i < kPer; ++i) {
        const uint32_t d = key[i * 64 + lane] - lo;
        const bool in = i * 64 + lane < cnt && (sp >= 32 || (d >> (sp & 31)) == fixed);
        if (in) atomicAdd(&hist[(d >> s) & dmask], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      // lane L holds bins 255 - 4L .. 252 - 4L, scanned from the top
      const uint4 h = reinterpret_cast<const uint4*>(hist)[63 - lane];
      const uint32_t c = h.x + h.y + h.z + h.w;
      const uint32_t incl = wave_inclusive_scan(c);
      uint32_t above = incl - c;
      const bool hit = above < k && k <= incl;
      const uint64_t hm = __ballot(hit);
      uint32_t bin = 0u, nbin = 0u;
      if (hit) {
        const uint32_t hv[4] = {h.w, h.z, h.y, h.x};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above + hv[q] >= k) {
            bin = 255u - 4u * (uint32_t)lane - (uint32_t)q;
            nbin = hv[q];
            break;
          }
          above += hv[q];
        }
      }
      const int src = __ffsll((unsigned long long)hm) - 1;
      bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
      nbin = (uint32_t)__builtin_amdgcn_readlane((int)nbin, src);
      above = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
      if (!exact && sp >= 32) {
        // first pass while scanning: keep the bin and everything above it when
        // that leaves room (the edge must be above key 0 to serve as threshold)
        edge = lo + (bin << s);
        if (edge == 0x7FFFFFFFu) edge = 0x7FFFFFFEu;  // (no key takes the value of -0's pre-key)
        if (edge > 0u && (int)(above + nbin) <= kCap - kRoom) {
          approx = true;
          break;
        }
      }
      k -= above;
      fixed = (sp >= 32 ? 0u : (fixed << ((sp - s) & 31))) | bin;
      sp = s;
      if (s == 0) break;
      s = max(0, s - 8);
    }
    const uint32_t t = approx ? edge : lo + fixed;  // approx: keep keys >= t; exact: the K-th largest
    // ---- stable compaction in place: an element only moves down, and the
    // writes of step i land below element 64 (i + 1), so step i reads its
    // elements before any write can reach them
    __builtin_amdgcn_wave_barrier();
    int out = 0;
    uint32_t eq_seen = 0u;
#pragma unroll 2
    for (int i = 0; i < kPer; ++i) {
      const bool pres = i * 64 + lane < cnt;
      const uint32_t kv = key[i * 64 + lane];
      const uint16_t j = idx[i * 64 + lane];
      const bool gt = pres && (approx ? kv >= t : kv > t);
      const bool eq = pres && !approx && kv == t;
      const uint64_t em = __ballot(eq);
      const bool keep = gt || (eq && eq_seen + lanes_below(em) < k);
      const uint64_t km = __ballot(keep);
      if (keep) {
        const int pos = out + (int)lanes_below(km);
        key[pos] = kv;
        idx[pos] = j;
      }
      out += __popcll(km);
      eq_seen += (uint32_t)__popcll(em);
    }
    __builtin_amdgcn_wave_barrier();
    cnt = out;
    nkey = out;
    // the next element is taken when its key > thr: at least K elements seen
    // have a key >= thr, all of them earlier (thr is a key, or an edge below
    // the K-th largest key that is not -0's pre-key)
    thr = t;
    thr_set = true;
  }
};

}  // namespace csa
