// hisparse.hip -- HiSparse-style staging of the selected compressed entries in a
// near (hot) pool ("Token 的一生：DSV4 架构与 DSpark" §5: the coordinator swaps
// this step's top-512 compressed tokens into fast storage and hands attention
// their indices there; entries that keep being selected stay near).
//
// Each sequence owns `hot` consecutive slots of the near pool. One workgroup
// per query row:
//   1. the row's selected entries are looked up in the sequence's residency
//      map (logical entry -> hot slot); hits are used in place and stamped
//      with this step, misses are ranked in selection order (ballots and one
//      workgroup scan, so the result does not depend on thread timing);
//   2. the victims are the `misses` least recently used slots among those not
//      used this step (empty slots first, equal stamps by lower slot): a top-k
//      radix select over the slots' keys, done by the same select as the top-512;
//   3. miss i takes victim i (both in ascending order), the maps are updated
//      (the victim's previous entry is unmapped), and every miss's entry is
//      copied from the far pool (through its page table) into its hot slot.
// The output is the near-pool slot of every selected entry, in the selection's
// order, ready for csa_sparse_attn over the near pool.
#include <limits.h>

#include "csa_device.hpp"
#include "csa_internal.hpp"
#include "topk_select.hpp"

namespace csa {
namespace {

constexpr int kHsThreads = 1024;
constexpr int kHsMaxHot = 4096;  // hot slots per sequence, at most
constexpr int kHsMaxSel = 512;   // selected entries per row, at most

template <int kE>
__global__ void __launch_bounds__(kHsThreads)
hisparse_swap_kernel(const int32_t* __restrict__ sel, int k, const int32_t* __restrict__ row_seq,
                     const uint8_t* __restrict__ f_lat, const float* __restrict__ f_sc,
                     const uint8_t* __restrict__ f_rope, const int32_t* __restrict__ f_pt,
                     int f_pt_stride, int f_ps, uint8_t* __restrict__ n_lat,
                     float* __restrict__ n_sc, uint8_t* __restrict__ n_rope, int lat_bytes,
                     int rope_bytes, int hot, int32_t* __restrict__ slot_of, int64_t max_entries,
                     int32_t* __restrict__ owner, int32_t* __restrict__ last_use, int step,
                     int32_t* __restrict__ near_idx) {
  __shared__ TopkLdsT<kHsMaxSel> L;
  __shared__ uint32_t s_used[kHsMaxHot / 32];
  __shared__ int32_t s_mj[kHsMaxSel], s_mpos[kHsMaxSel];
  __shared__ uint32_t s_red[kTopkMaxWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int s = row_seq[r];
  int32_t* const map = slot_of + (int64_t)s * max_entries;
  int32_t* const own = owner + (int64_t)s * hot;
  int32_t* const stamp = last_use + (int64_t)s * hot;
  for (int i = tid; i < kHsMaxHot / 32; i += kHsThreads) s_used[i] = 0u;
  for (int i = tid; i < kTopkBins; i += kHsThreads) L.hist[i] = 0u;
  __syncthreads();

  // ---- 1. hits in place, misses ranked by selection position (k <= 1024)
  int32_t j = -1, h = -1;
  if (tid < k) {
    j = sel[(int64_t)r * k + tid];
    if (j >= 0) h = map[j];
  }
  const bool miss = j >= 0 && h < 0;
  if (tid < k) {
    if (j < 0) {
      near_idx[(int64_t)r * k + tid] = -1;
    } else if (h >= 0) {
      atomicOr(&s_used[h >> 5], 1u << (h & 31));
      stamp[h] = step;
      near_idx[(int64_t)r * k + tid] = s * hot + h;
    }
  }
  const uint64_t bm = __ballot(miss);
  uint32_t nmiss;
  const uint32_t woff = wave_offsets<kHsThreads>((uint32_t)__popcll(bm), s_red, nmiss);
  if (miss) {
    const uint32_t rank = woff + (uint32_t)__popcll(bm & ((1ull << lane) - 1ull));
    s_mj[rank] = j;
    s_mpos[rank] = tid;
  }
  __syncthreads();  // s_used complete, miss list complete
  if (nmiss == 0) return;

  // ---- 2. victims: the nmiss largest keys over the hot slots (key 0: used
  // this step, never taken; empty slots largest; then older stamps larger)
  const int seg = wave * 64 * kE;
  uint32_t kr[kE];
#pragma unroll
  for (int i = 0; i < kE; ++i) {
    const int e = seg + 64 * i + lane;
    uint32_t key = 0u;
    if (e < hot && !((s_used[e >> 5] >> (e & 31)) & 1u)) {
      const int32_t o = own[e];
      key = o < 0 ? 0xFFFFFFFFu : 0xFFFFFFFEu - (uint32_t)max(stamp[e], 0);
    }
    kr[i] = key;
  }
  topk_select<kE, kHsThreads>(kr, hot, (int)nmiss, seg, L);

  // ---- 3. miss i -> victim i: maps, stamp, output slot
  if (tid < (int)nmiss) {
    const int v = L.out_e[tid];
    const int32_t jm = s_mj[tid];
    const int32_t old = own[v];
    if (old >= 0) map[old] = -1;
    own[v] = jm;
    map[jm] = v;
    stamp[v] = step;
    near_idx[(int64_t)r * k + s_mpos[tid]] = s * hot + v;
  }
  // ---- copies: 16-byte pieces of each miss's latent, RoPE dims and scale
  const int lat_q = lat_bytes / 16, rope_q = rope_bytes / 16;
  const int per = lat_q + rope_q + (f_sc ? 1 : 0);
  for (int w = tid; w < (int)nmiss * per; w += kHsThreads) {
    const int i = w / per, q = w % per;
    const int32_t jm = s_mj[i];
    const int v = L.out_e[i];
    const int64_t fs = (int64_t)f_pt[(int64_t)s * f_pt_stride + jm / f_ps] * f_ps + jm % f_ps;
    const int64_t ns = (int64_t)s * hot + v;
    if (q < lat_q) {
      reinterpret_cast<uint4*>(n_lat + ns * lat_bytes)[q] =
          reinterpret_cast<const uint4*>(f_lat + fs * lat_bytes)[q];
    } else if (q < lat_q + rope_q) {
      reinterpret_cast<uint4*>(n_rope + ns * rope_bytes)[q - lat_q] =
          reinterpret_cast<const uint4*>(f_rope + fs * rope_bytes)[q - lat_q];
    } else {
      n_sc[ns] = f_sc[fs];
    }
  }
}

}  // namespace

int hisparse_max_hot() { return kHsMaxHot; }
int hisparse_max_sel() { return kHsMaxSel; }

hipError_t launch_hisparse_swap(const int32_t* sel, int R, int k, const int32_t* row_seq,
                                const csa_kv_pool& far, const int32_t* far_pt, int far_pt_stride,
                                const csa_kv_pool& near, int hot, int32_t* slot_of,
                                int64_t max_entries, int32_t* owner, int32_t* last_use, int step,
                                int32_t* near_idx, hipStream_t s) {
  if (R == 0) return hipSuccess;
  const bool f32 = far.fmt == CSA_F32;
  const int lat_bytes = kLatent * (f32 ? 4 : 1);
  const int rope_bytes = kRope * (f32 ? 4 : 2);
  const int e = hot <= 1024 ? 1 : (hot <= 2048 ? 2 : 4);
#define CSA_HS(E)                                                                                 \
  hipLaunchKernelGGL((hisparse_swap_kernel<E>), dim3(R), dim3(kHsThreads), 0, s, sel, k, row_seq,  \
                     (const uint8_t*)far.latent, f32 ? nullptr : far.latent_scale,                 \
                     (const uint8_t*)far.rope, far_pt, far_pt_stride, far.page_size,              \
                     (uint8_t*)near.latent, f32 ? nullptr : near.latent_scale,                    \
                     (uint8_t*)near.rope, lat_bytes, rope_bytes, hot, slot_of, max_entries, owner, \
                     last_use, step, near_idx)
  if (e == 1) CSA_HS(1);
  else if (e == 2) CSA_HS(2);
  else CSA_HS(4);
#undef CSA_HS
  return hipGetLastError();
}

}  // namespace csa
