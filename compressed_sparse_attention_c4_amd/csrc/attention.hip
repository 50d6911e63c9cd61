// attention.hip -- MLA-style multi-query attention over gathered KV entries:
// CSA (the selected compressed entries plus the raw sliding window) and HCA
// (every visible heavily compressed entry plus the window).
//
// "Token 的一生：DSV4 架构与 DSpark" §1: attention reads only the 512 selected
// compressed KV; "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）" CSA paragraph (sliding
// window branch for recent uncompressed tokens), HCA paragraph (dense attention
// over ~128x compressed blocks), "低精度與儲存策略的配合" (FP8 latent, BF16 RoPE).
//
// All H query heads share each 576-dim entry (512 latent + 64 RoPE; the value
// is the latent part), so per query the work is two dense contractions,
// S = Q K^T and O = P V, run on bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
// e4m3 codes are exact in bf16, so the per-entry FP8 scale is applied to the
// latent score term and folded into P for the value product.
//
// A workgroup owns one query and a contiguous range of its entry list; a pair
// of waves owns 16 heads (one wave scores half of each tile's entries and
// accumulates half of the value dims). Entries are gathered 32 at a time:
// each thread loads 32 code bytes of one entry, converts them with
// v_cvt_scalef32_pk_bf16_fp8 and writes them row-major to one of two LDS
// tiles; S reads K fragments from the tile and P V reads the value fragments
// from the same tile with ds_read_b64_tr_b16. A tile's gathers are issued two
// tiles ahead of its matrix work. An online softmax runs over the tiles. Long
// entry lists are split over several workgroups whose partial (max, sum, O)
// are merged by a second kernel.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kTile = 32;             // entries per LDS tile
constexpr int kKStride = kKvDim + 8;  // bf16 elements per row of the K tile
constexpr int kPStride = kTile + 8;   // bf16 elements per row of P
constexpr int kMaxSplit = 1024;       // entries one workgroup handles, at most

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_bf16(const v4i& a, const v4i& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Entry list of one query: n1 compressed entries then n2 window entries.
struct EntryList {
  int n1, n2, w0;  // w0 = first window position
};

__device__ __forceinline__ EntryList entry_list(int p, int k_sel, bool hca, int ratio, int window) {
  EntryList L;
  L.n1 = hca ? (p + 1) / ratio : k_sel;
  L.w0 = max(0, p - window + 1);
  L.n2 = p + 1 - L.w0;
  return L;
}

// Slot (and pool: 0 compressed, 1 raw) of entry i, or -1 when masked.
__device__ __forceinline__ int64_t entry_slot(int i, const EntryList& L, int t, int seq,
                                              bool hca, const int32_t* phys_idx, int k_sel,
                                              const int32_t* comp_pt, int comp_pt_stride,
                                              int comp_ps, const int32_t* raw_pt,
                                              int raw_pt_stride, int raw_ps, int& pool) {
  if (i < L.n1) {
    pool = 0;
    if (!hca) return (int64_t)phys_idx[(int64_t)t * k_sel + i];
    return (int64_t)comp_pt[(int64_t)seq * comp_pt_stride + i / comp_ps] * comp_ps + i % comp_ps;
  }
  pool = 1;
  if (i < L.n1 + L.n2) {
    const int pos = L.w0 + (i - L.n1);
    return (int64_t)raw_pt[(int64_t)seq * raw_pt_stride + pos / raw_ps] * raw_ps + pos % raw_ps;
  }
  return -1;
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only (not for its outstanding global loads, as __syncthreads would), then
// s_barrier.
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Entry -> pool choice as 64-bit masks (bitwise selects keep gathers
// straight-line; masked entries read a stand-in and are zeroed).
struct Pick {
  int64_t slot;
  uint64_t mc, mr, md;
};
__device__ __forceinline__ Pick pick_of(int es) {
  Pick k;
  k.slot = es >= 0 ? (es >> 1) : 0;
  k.md = es < 0 ? ~0ull : 0ull;
  k.mr = (es >= 0 && (es & 1)) ? ~0ull : 0ull;
  k.mc = ~(k.md | k.mr);
  return k;
}
__device__ __forceinline__ uint64_t pick_base(const Pick& k, const void* c, const void* r,
                                              const void* d) {
  return ((uint64_t)c & k.mc) | ((uint64_t)r & k.mr) | ((uint64_t)d & k.md);
}
// A load from a device address held as an integer, as a global-memory load
// (a plain pointer made from an integer is generic, and generic loads count
// in the LDS counter too, so every LDS wait would also wait for them).
template <class V>
__device__ __forceinline__ V gload(uint64_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(1))) V*>(addr);
}

// A row of zeros as long as an entry's latent codes. A masked entry's gathers
// read from here (slot 0), so they load zeros and need no select afterwards;
// a select on a prefetched value would make the compiler wait for that load
// where the select lands, in the middle of the matrix work.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kLatent] = {};

// Workgroup coordinates (a = split, chunk, value slice or head; t = query; z =
// head block) from a 1-D grid that groups each query's workgroups by XCD.
// Workgroup b runs on XCD b % 8; with g = min(8, T rounded up to a power of
// two), query t gets the workgroups with b % g == t % g, i.e. 8 / g XCDs
// (one when T >= 8). The query's operands, P' and the cache lines its value
// slices share are then fetched into those XCDs' L2 only, not into all eight.
// b past the last query maps to t >= T, which the kernels skip.
struct Coord {
  int a, t, z;
};
__device__ __forceinline__ Coord block_coord(int na, int nz, int g) {
  const int b = blockIdx.x;
  int r = b / g;
  const int a = r % na;
  r /= na;
  return {a, (r / nz) * g + b % g, r % nz};
}
int xcd_group(int T) {
  int g = 1;
  while (g < T && g < 8) g *= 2;
  return g;
}
dim3 xcd_grid(int na, int nz, int T) {
  const int g = xcd_group(T);
  return dim3((unsigned)(g * na * nz * ((T + g - 1) / g)));
}

// Two e4m3 codes (bytes 0,1 or 2,3 of w) -> two bf16 (exact), one instruction.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// The two pools are passed as plain pointers so that the per-entry choice
// between them is a register select (a struct chosen at run time would be
// copied to private memory).
// The two contractions of a tile split over pairs of waves: pair g owns heads
// 16g..16g+15 of the workgroup's head block; within a pair, wave `half`
// scores entries 16*half..+15 of each tile and accumulates value dims
// 256*half..+255. A wave then holds a 16 x 256 output block (64 accumulators
// per lane) instead of 16 x 512, which leaves registers for the LDS operand
// reads to run ahead of the matrix ops, and two waves share each SIMD, so one
// wave's LDS and softmax latency hides behind the other's matrix work. The
// two waves of a pair exchange their tile maxima and write the two halves of
// the tile's P through LDS.
//
// Per tile, the vector ALU is the scarce unit (a wave64 VALU op issues over
// four cycles, a tile's matrix work is 34 MFMAs per wave), so the staging is
// built to need few VALU ops: a thread gathers 32 contiguous code bytes of one
// entry (one address per tile), the K tile is stored once, row-major, and the
// value operand of P V is read from it with the transposing LDS load; the
// softmax keeps its row sums per lane until the end and rescales O only when
// a head's maximum grows by more than kRescaleSlack.
constexpr float kRescaleSlack = 8.f;  // p = exp(s - m_ref) <= e^8 between rescales

template <int kHG, bool kOutF32>
__global__ void __launch_bounds__(kHG * 128)
attn_mfma_kernel(const uint16_t* __restrict__ q, int H, const int32_t* __restrict__ q_seq,
                 const int32_t* __restrict__ q_pos, bool hca, const int32_t* __restrict__ phys_idx,
                 int k_sel, int ratio, const uint8_t* __restrict__ c_lat,
                 const float* __restrict__ c_sc, const uint16_t* __restrict__ c_rope, int c_ps,
                 const int32_t* __restrict__ comp_pt, int comp_pt_stride,
                 const uint8_t* __restrict__ r_lat, const float* __restrict__ r_sc,
                 const uint16_t* __restrict__ r_rope, int r_ps, const int32_t* __restrict__ raw_pt,
                 int raw_pt_stride, int window, float scale, void* __restrict__ out,
                 float* __restrict__ part, int split_len, int nsplit, int T, int nz, int g,
                 int2* __restrict__ qsplit) {
  constexpr int kThreads = kHG * 128;
  // Two K tiles (the one being computed and the next), row-major bf16
  // [entry][576]: latent codes as exact bf16, then the RoPE dims.
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_p[kHG][16 * kPStride];
  __shared__ float s_scale[2][kTile];
  __shared__ int s_valid[2][kTile];
  __shared__ __attribute__((aligned(16))) float s_mx[kHG][2][16];  // per pair and half: a value per head
  __shared__ int32_t s_eslot[kMaxSplit];  // entry slots of this split: slot*2 + pool, -1 masked

  // Uniform splits (qsplit null): query t's list is cut into nsplit pieces of
  // split_len entries. Balanced (qsplit set, one head block, T <= 64): the
  // grid's nsplit workgroups are shared out in proportion to the queries'
  // list lengths, every workgroup deriving the same assignment: a piece of
  // `target` entries each, target = the smallest multiple of a tile that
  // leaves at most nsplit pieces; query t owns workgroups off_t .. off_t +
  // ceil(len_t / target) - 1, and workgroup 0 records (off_t, count) for the
  // combine.
  Coord bc;
  int t, split, e_len;
  if (qsplit) {
    __shared__ int s_off[65];
    __shared__ int s_len[64];
    __shared__ int s_target;
    if (threadIdx.x < 64) {
      int n = 0;
      if ((int)threadIdx.x < T) {
        const EntryList Lq = entry_list(q_pos[threadIdx.x], k_sel, hca, ratio, window);
        n = Lq.n1 + Lq.n2;
      }
      s_len[threadIdx.x] = n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t sum = 0;
      for (int i = 0; i < T; ++i) sum += s_len[i];
      const int64_t free_slots = nsplit - T;  // >= 1: the host sizes the grid
      int64_t target = (sum + free_slots - 1) / free_slots;
      target = (target + kTile - 1) / kTile * kTile;
      target = target < kTile ? kTile : (target > kMaxSplit ? kMaxSplit : target);
      int off = 0;
      for (int i = 0; i < T; ++i) {
        s_off[i] = off;
        off += (int)((s_len[i] + target - 1) / target);
      }
      s_off[T] = off;
      s_target = (int)target;
    }
    __syncthreads();
    const int w = blockIdx.x;
    if (w == 0 && (int)threadIdx.x < T)
      qsplit[threadIdx.x] = make_int2(s_off[threadIdx.x], s_off[threadIdx.x + 1] - s_off[threadIdx.x]);
    if (w >= s_off[T]) return;  // past the last piece (uniform across the workgroup)
    int tq = 0;
    while (tq + 1 < T && s_off[tq + 1] <= w) ++tq;
    t = tq;
    split = w - s_off[tq];
    e_len = s_target;
    bc = Coord{split, t, 0};
  } else {
    bc = block_coord(nsplit, nz, g);
    t = bc.t;
    if (t >= T) return;
    split = bc.a;
    e_len = split_len;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 1, half = wave & 1;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int seq = q_seq[t];
  const int p = q_pos[t];
  const EntryList L = entry_list(p, k_sel, hca, ratio, window);
  const int total = L.n1 + L.n2;
  const int e_begin = split * e_len;
  const int e_end = min(total, e_begin + e_len);
  const int n_split = max(0, e_end - e_begin);

  // Heads of this pair: hbase .. hbase+15.
  const int hbase = bc.z * kHG * 16 + hg * 16;
  // Query operand (A): head hbase + col, dims step*32 + grp*8 .. +7.
  v4i qa[18];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + hbase + col) * kKvDim + grp * 8;
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      uint4 x = *reinterpret_cast<const uint4*>(qrow + s * 32);
      qa[s] = v4i{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
    }
  }

  // m: the reference maximum of each head (rows 4*grp + r); l: this lane's
  // share of the row sum (its entry column, summed over the tiles).
  float m[4], l[4];
  v4f o[16];  // dims 256*half + 16n + col, rows = heads 4*grp + r
#pragma unroll
  for (int r = 0; r < 4; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
#pragma unroll
  for (int n = 0; n < 16; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  // Slots of every entry of this split, resolved once (one round of
  // page-table / index reads for the whole split, all threads in parallel), so
  // the tile gathers below depend on LDS only.
  for (int i = tid; i < n_split; i += kThreads) {
    int pool = 0;
    const int64_t slot = entry_slot(e_begin + i, L, t, seq, hca, phys_idx, k_sel, comp_pt,
                                    comp_pt_stride, c_ps, raw_pt, raw_pt_stride, r_ps, pool);
    s_eslot[i] = slot >= 0 ? (int32_t)(slot * 2 + pool) : -1;
  }
  __syncthreads();

  // Staging tasks: entry e = task / 16 of the tile, part c = task % 16: latent
  // codes 8c + 128j .. +7 (j < 4), RoPE chunk c % 8 (16 B; written by c < 8)
  // and the entry's FP8 scale (written by c == 0). A masked entry, or one past
  // the split, reads the zero row.
  constexpr int kTasks = (kTile * 16) / kThreads;
  v2i lat[kTasks][4];
  v4i rope[kTasks];
  float esc[kTasks];
  int evalid[kTasks];
  const uint8_t* zero = g_zero_row;
  const int last = max(n_split - 1, 0);  // clamped LDS index: reads stay unconditional
  auto issue_loads = [&](int tile0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kTasks; ++k) {
      const int task = tid + k * kThreads;
      const int e = task >> 4, c = task & 15;
      const int li = tile0 - e_begin + e;
      const int es = s_eslot[min(li, last)];
      const Pick pk = pick_of(li < n_split ? es : -1);
      evalid[k] = !pk.md;
      const uint64_t lb = pick_base(pk, c_lat, r_lat, zero) + pk.slot * kLatent + 8 * c;
#pragma unroll
      for (int j = 0; j < 4; ++j) lat[k][j] = gload<v2i>(lb + 128 * j);
      rope[k] = gload<v4i>(pick_base(pk, c_rope, r_rope, zero) + pk.slot * (kRope * 2) + 16 * (c & 7));
      esc[k] = gload<float>(pick_base(pk, c_sc, r_sc, zero) + pk.slot * 4);
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kTasks; ++k) {
      const int task = tid + k * kThreads;
      const int e = task >> 4, c = task & 15;
      uint16_t* row = &s_k[buf][e * kKStride];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0 = (uint32_t)lat[k][j][0], w1 = (uint32_t)lat[k][j][1];
        *reinterpret_cast<uint4*>(row + 8 * c + 128 * j) =
            make_uint4(fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
                       fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1));
      }
      if (c < 8)
        *reinterpret_cast<uint4*>(row + kLatent + 8 * c) =
            make_uint4((uint32_t)rope[k][0], (uint32_t)rope[k][1], (uint32_t)rope[k][2],
                       (uint32_t)rope[k][3]);
      if (c == 0) {
        s_scale[buf][e] = esc[k];
        s_valid[buf][e] = evalid[k];
      }
    }
  };

  const int n_tiles = (n_split + kTile - 1) / kTile;
  issue_loads(e_begin);
  stage(0);
  issue_loads(e_begin + kTile);
  lds_sync();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const uint16_t* kt = s_k[buf];
    // ---- S = Q K^T for 16 heads x the 16 entries of this half. The K
    // fragments are read ahead (six in flight), so the matrix cores do not
    // wait out an LDS round trip per step.
    const int e = half * 16 + col;
    v4i kf[18];
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      const uint4 kk = *reinterpret_cast<const uint4*>(&kt[e * kKStride + s * 32 + grp * 8]);
      kf[s] = v4i{(int)kk.x, (int)kk.y, (int)kk.z, (int)kk.w};
    }
    v4f acc_l = {0.f, 0.f, 0.f, 0.f}, acc_r = acc_l;
#pragma unroll
    for (int s = 0; s < 16; ++s) acc_l = mfma_bf16(qa[s], kf[s], acc_l);
    acc_r = mfma_bf16(qa[16], kf[16], acc_r);
    acc_r = mfma_bf16(qa[17], kf[17], acc_r);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    const bool valid = s_valid[buf][e] != 0;
    const float sc = s_scale[buf][e];
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = valid ? scale * fmaf(sc, acc_l[r], acc_r[r]) : -INFINITY;
    // ---- tile maxima of the pair (rows = heads 4*grp + r)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mh = row16_max(sv[r]);
      if (col == 0) s_mx[hg][half][grp * 4 + r] = mh;
    }
    lds_sync();
    const float4 mx0 = *reinterpret_cast<const float4*>(&s_mx[hg][0][grp * 4]);
    const float4 mx1 = *reinterpret_cast<const float4*>(&s_mx[hg][1][grp * 4]);
    const float mt[4] = {fmaxf(mx0.x, mx1.x), fmaxf(mx0.y, mx1.y), fmaxf(mx0.z, mx1.z),
                         fmaxf(mx0.w, mx1.w)};
    // Both waves of the pair see the same maxima, so they take the same
    // rescale decisions. A head moves its reference maximum only when the
    // tile's exceeds it by more than the slack (always, the first time).
    bool grow = false;
    float corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool up = mt[r] > m[r] + kRescaleSlack;
      corr[r] = up ? __expf(m[r] - mt[r]) : 1.f;  // m = -inf: 0
      m[r] = up ? mt[r] : m[r];
      grow |= up;
      const float pr = sv[r] == -INFINITY ? 0.f : __expf(sv[r] - m[r]);
      l[r] = fmaf(l[r], corr[r], pr);
      // P' = p * (value dequant scale), bf16, stored row-major [head][entry]
      s_p[hg][(grp * 4 + r) * kPStride + e] = f32_to_bf16(pr * sc);
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int n = 0; n < 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[n][r] *= corr[r];
    }
    lds_sync();  // both halves of P written
    // ---- O += P V: A = P (head col, entries grp*8..+7); B = V (entries
    // grp*8..+7, dim col of block n) read from the K tile with the
    // transposing load: in each 16-lane group, lane j receives element j % 4
    // of the 4-element rows fetched by lanes 4k + j/4 (k = 0..3), so lane
    // 4a + b fetches entry 8*grp + 4h + a, dims 4b..4b+3 of the block.
    const uint4 pa8 = *reinterpret_cast<const uint4*>(&s_p[hg][col * kPStride + grp * 8]);
    const v4i pa = v4i{(int)pa8.x, (int)pa8.y, (int)pa8.z, (int)pa8.w};
    const uint16_t* vb = kt + (8 * grp + (col >> 2)) * kKStride + half * 256 + 4 * (col & 3);
    v4i vf[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const v2i lo = __builtin_bit_cast(
          v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) v4s*)(vb + n * 16)));
      const v2i hi = __builtin_bit_cast(
          v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) v4s*)(vb + 4 * kKStride + n * 16)));
      vf[n] = v4i{lo[0], lo[1], hi[0], hi[1]};
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) o[n] = mfma_bf16(pa, vf[n], o[n]);
    __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // ---- the next tile (its gathers landed during this one) into the other
    // buffer, then the gathers of the tile after it (past the split: zero
    // rows, never used; no branch, so the waits stay exact)
    stage(buf ^ 1);
    issue_loads(e_begin + (it + 2) * kTile);
    lds_sync();  // next tile and P free
  }

  // the row sums: over the lanes of each row, then the two halves
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = row16_sum(l[r]);
    if (col == 0) s_mx[hg][half][grp * 4 + r] = lr;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) l[r] = s_mx[hg][0][grp * 4 + r] + s_mx[hg][1][grp * 4 + r];

  const int h0 = hbase + grp * 4;
  const int d0 = half * 256 + col;
  if (nsplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
      const int64_t obase = ((int64_t)t * H + h0 + r) * kLatent + d0;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const float v = o[n][r] * inv;
        if (kOutF32) reinterpret_cast<float*>(out)[obase + n * 16] = v;
        else reinterpret_cast<uint16_t*>(out)[obase + n * 16] = f32_to_bf16(v);
      }
    }
  } else {
    // partials: [slot][H][512] O, then [slot][H] m and l (O and l are
    // relative to m); slot = t * nsplit + split (uniform) or the workgroup
    // (balanced, nsplit slots in all). O is fp32 for fp32 output and bf16
    // for bf16 output (the merge reads half the bytes; the rounding adds at
    // most 2^-9 of the largest value to the output, beside P's 2^-9), in the
    // front of the fp32-sized region.
    const int64_t nslot = qsplit ? nsplit : (int64_t)T * nsplit;
    const int64_t ph = (qsplit ? (int64_t)blockIdx.x : (int64_t)t * nsplit + split) * H;
    float* po = part;
    float* pm = part + nslot * H * kLatent;
    float* pl = pm + nslot * H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t obase = (ph + h0 + r) * kLatent + d0;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        if (kOutF32) po[obase + n * 16] = o[n][r];
        else reinterpret_cast<uint16_t*>(po)[obase + n * 16] = f32_to_bf16(o[n][r]);
      }
      if (col == 0 && half == 0) {
        pm[ph + h0 + r] = m[r];
        pl[ph + h0 + r] = l[r];
      }
    }
  }
}

// Element i of the O partials: fp32, or bf16 for bf16 output.
template <bool kF32>
__device__ __forceinline__ float part_o(const float* part, int64_t i) {
  return kF32 ? part[i] : bf16_to_f32(reinterpret_cast<const uint16_t*>(part)[i]);
}

template <bool kOutF32>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part, int T, int H, int nsplit,
                    void* __restrict__ out, int g, const int2* __restrict__ qsplit) {
  // four heads per workgroup, one wave each; a lane holds 8 of the 512 dims
  const Coord bc = block_coord(H / 4, 1, g);  // on the XCDs that wrote the query's partials
  const int t = bc.t, h = bc.a * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  // the query's slots: t * nsplit .. + nsplit (uniform) or qsplit[t] (balanced)
  const int64_t nslot = qsplit ? nsplit : (int64_t)T * nsplit;
  int64_t s0 = (int64_t)t * nsplit;
  int ns = nsplit;
  if (qsplit) {
    const int2 q = qsplit[t];
    s0 = q.x;
    ns = q.y;
  }
  const float* pm = part + nslot * H * kLatent;
  const float* pl = pm + nslot * H;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pm[(s0 + s) * H + h]);
  float Lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // branch-free, so that the loads of several slots are in flight together
  // (an empty slot's partial is written as zeros, and its factor is 0)
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const int64_t idx = (s0 + s) * H + h;
    const float ms = pm[idx];
    const float f = ms == -INFINITY ? 0.f : __expf(ms - M);
    Lsum = fmaf(pl[idx], f, Lsum);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(part_o<kOutF32>(part, idx * kLatent + lane + 64 * k), f, acc[k]);
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int64_t ob = ((int64_t)t * H + h) * kLatent + lane;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (kOutF32) reinterpret_cast<float*>(out)[ob + 64 * k] = acc[k] * inv;
    else reinterpret_cast<uint16_t*>(out)[ob + 64 * k] = f32_to_bf16(acc[k] * inv);
  }
}

// The merge for length-balanced splits, where a long list owns many slots
// (HCA over ragged lengths: the longest of 16 lists takes ~50 of 256): one
// head per workgroup, its slots dealt round-robin to the four waves, whose
// partial sums meet in LDS. A wave then walks a quarter of the slots, so the
// longest list's merge is four times shorter than with one wave per head.
template <bool kOutF32>
__global__ void __launch_bounds__(256)
attn_combine_slots_kernel(const float* __restrict__ part, int T, int H, int nslot,
                          void* __restrict__ out, int g, const int2* __restrict__ qsplit) {
  __shared__ float s_acc[4][kLatent];
  __shared__ float s_red[8];
  const Coord bc = block_coord(H, 1, g);
  const int t = bc.t, h = bc.a;
  if (t >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int2 qs = qsplit[t];
  const int64_t s0 = qs.x;
  const int ns = qs.y;
  const float* pm = part + (int64_t)nslot * H * kLatent;
  const float* pl = pm + (int64_t)nslot * H;
  // the query's maximum over its slots (every wave, lanes over the slots)
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, pm[(s0 + s) * H + h]);
  M = wave_max(M);
  float Lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // branch-free within a wave's turn, so that the loads of several slots are
  // in flight together (an empty slot's partial is zeros, its factor 0)
#pragma unroll 4
  for (int s = wave; s < ns; s += 4) {
    const int64_t idx = (s0 + s) * H + h;
    const float ms = pm[idx];
    const float f = ms == -INFINITY ? 0.f : __expf(ms - M);
    Lsum = fmaf(pl[idx], f, Lsum);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(part_o<kOutF32>(part, idx * kLatent + lane + 64 * k), f, acc[k]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) s_acc[wave][lane + 64 * k] = acc[k];
  if (lane == 0) s_red[wave] = Lsum;
  __syncthreads();
  const float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int64_t ob = ((int64_t)t * H + h) * kLatent;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int d = tid + 256 * k;
    const float v = ((s_acc[0][d] + s_acc[1][d]) + (s_acc[2][d] + s_acc[3][d])) * inv;
    if (kOutF32) reinterpret_cast<float*>(out)[ob + d] = v;
    else reinterpret_cast<uint16_t*>(out)[ob + d] = f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Two-phase path for few queries (decode). With T small, the split kernel
// needs many splits per query and each writes a 64 x 512 fp32 partial, more
// bytes than the KV it reads. Here phase A computes, for each chunk (64 or 96
// entries, two_phase_chunk) of a query's entry list, all heads' scores, the chunk's softmax max m_c and
// sum l_c, and the weights P' = exp(s - m_c) * (value FP8 scale) in bf16;
// phase B merges the chunks' (m_c, l_c) into the exact normaliser and sums
// f_c * (P' V) for one 64-dim slice of the value, f_c = exp(m_c - M) / L. No
// merge follows. Phase B gets its values one of two ways:
//  - copy: phase A also writes the latent codes it gathered into one
//    contiguous [entry][64] block per value slice, so phase B reads values,
//    weights and statistics in a single round of independent loads;
//  - gather: phase A stores each entry's slot, and phase B gathers its
//    64-byte value slices straight from the pools (one round of loads for
//    statistics, slots and weights, then one round of gathers).
// The copy costs phase A 512 B of writes per entry, and a kernel's written
// lines are flushed from L2 before the next kernel starts, so with many
// queries (a copy of several MB) the gather is faster; with few, the copy's
// single round is.
constexpr int kChunk = 64;                // entries per phase-A workgroup (or kChunkWide)
constexpr int kChunkWide = 96;
constexpr int kAttnCUs = 256;             // CUs of the GPU (32 per XCD)
constexpr int kSlice = 64;                // value dims per phase-B workgroup
constexpr int kTwoPhaseMaxE = 768;        // entry lists up to this length
constexpr int kVStride = kSlice + 8;      // bf16 per value row in phase B's LDS
constexpr size_t kGatherMinCopy = 4u << 20;  // value copies this large take the gather

template <int kCh>
__global__ void __launch_bounds__(256)
attn_scores_kernel(const uint16_t* __restrict__ q, int H, const int32_t* __restrict__ q_seq,
                   const int32_t* __restrict__ q_pos, bool hca, const int32_t* __restrict__ phys_idx,
                   int k_sel, int ratio, const uint8_t* __restrict__ c_lat,
                   const float* __restrict__ c_sc, const uint16_t* __restrict__ c_rope, int c_ps,
                   const int32_t* __restrict__ comp_pt, int comp_pt_stride,
                   const uint8_t* __restrict__ r_lat, const float* __restrict__ r_sc,
                   const uint16_t* __restrict__ r_rope, int r_ps,
                   const int32_t* __restrict__ raw_pt, int raw_pt_stride, int window, float scale,
                   uint16_t* __restrict__ pw, float2* __restrict__ stats,
                   uint8_t* __restrict__ vcopy, int32_t* __restrict__ ent, int e_pad, int T,
                   int nz, int g) {
  constexpr int kCB = kCh / 16;  // 16-entry column blocks of the chunk
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kCh * kKStride];
  __shared__ int32_t s_es[kCh];
  __shared__ float s_sc[kCh];
  __shared__ uint64_t s_la[kCh], s_ra[kCh];  // latent / RoPE row addresses
  const int n_chunks = e_pad / kCh;
  const Coord bc = block_coord(n_chunks, nz, g);
  const int chunk = bc.a, t = bc.t;
  if (t >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int e0 = chunk * kCh;
  // A selected entry's slot needs nothing of the query's position: its load
  // goes out together with the position's, one round trip earlier than a
  // lookup that waits for the entry list.
  int32_t pre = -1;
  if (!hca && tid < kCh && e0 + tid < k_sel) pre = phys_idx[(int64_t)t * k_sel + e0 + tid];
  const int seq = q_seq[t], p = q_pos[t];
  const EntryList L = entry_list(p, k_sel, hca, ratio, window);
  const int total = min(L.n1 + L.n2, e_pad);  // a list longer than the stated bound is cut
  const int hb0 = bc.z * 64;
  // phase B's value source (copy mode: vcopy set, ent null; gather: the reverse)
  uint8_t* vc_t = vcopy + (int64_t)t * (kLatent / kSlice) * e_pad * kSlice;
  int32_t* ent_t = ent + (int64_t)t * e_pad + e0;
  if (e0 >= total) {
    // past this query's list: zero weights, dead statistics and masked
    // entries, so that phase B reads every chunk without knowing the list's
    // length
    const int hh = tid >> 2, part = tid & 3;  // head, quarter of the chunk
    v4i* prow = reinterpret_cast<v4i*>(pw + ((int64_t)t * H + hb0 + hh) * e_pad + e0 + part * (kCh / 4));
#pragma unroll
    for (int k = 0; k < kCh / 32; ++k) prow[k] = v4i{0, 0, 0, 0};
    if (tid < 64) stats[((int64_t)t * H + hb0 + tid) * n_chunks + chunk] = make_float2(-INFINITY, 0.f);
    if (bc.z == 0) {
      if (ent) {
        if (tid < kCh) ent_t[tid] = -1;
      } else {
#pragma unroll
        for (int k = 0; k < kCh / 8; ++k) {
          const int idx = tid + k * 256, e = idx >> 5, c = idx & 31;
          *reinterpret_cast<v4i*>(vc_t + ((int64_t)(c >> 2) * e_pad + e0 + e) * kSlice + 16 * (c & 3)) =
              v4i{0, 0, 0, 0};
        }
      }
    }
    return;
  }
  const int hbase = hb0 + wave * 16;
  float scv = 0.f;
  if (tid < kCh) {
    const int i = e0 + tid;
    int pool = 0;
    int64_t slot = -1;
    if (i < total) {
      if (!hca && i < L.n1) slot = pre;
      else
        slot = entry_slot(i, L, t, seq, hca, phys_idx, k_sel, comp_pt, comp_pt_stride, c_ps,
                          raw_pt, raw_pt_stride, r_ps, pool);
    }
    const int32_t w = slot >= 0 ? (int32_t)(slot * 2 + pool) : -1;
    s_es[tid] = w;
    if (bc.z == 0 && ent) ent_t[tid] = w;  // the entries' slots for phase B's gathers
    // every gather of the entry starts from these (masked: the zero row)
    const Pick pk = pick_of(w);
    s_la[tid] = pick_base(pk, c_lat, r_lat, g_zero_row) + pk.slot * kLatent;
    s_ra[tid] = pick_base(pk, c_rope, r_rope, g_zero_row) + pk.slot * (kRope * 2);
    scv = gload<float>(pick_base(pk, c_sc, r_sc, g_zero_row) + pk.slot * 4);
  }
  // the query operand is loaded after the slot reads, so that waiting for
  // those does not wait for these
  __builtin_amdgcn_sched_barrier(0);
  v4i qa[18];
  {
    const uint16_t* qrow = q + ((int64_t)t * H + hbase + col) * kKvDim + grp * 8;
#pragma unroll
    for (int s = 0; s < 18; ++s) qa[s] = *reinterpret_cast<const v4i*>(qrow + s * 32);
  }
  lds_sync();
  // gathers: kCh entries x 32 latent chunks of 16 B (kCh / 8 per thread, one
  // entry row per 32 lanes), kCh x 8 RoPE chunks (kCh / 32 per thread)
  v4i lat[kCh / 8], rp[kCh / 32];
#pragma unroll
  for (int k = 0; k < kCh / 8; ++k) {
    const int idx = tid + k * 256, e = idx >> 5, c = idx & 31;
    lat[k] = gload<v4i>(s_la[e] + 16 * c);
  }
#pragma unroll
  for (int k = 0; k < kCh / 32; ++k) {
    const int idx = tid + k * 256, e = idx >> 3, c = idx & 7;
    rp[k] = gload<v4i>(s_ra[e] + 16 * c);
  }
#pragma unroll
  for (int k = 0; k < kCh / 8; ++k) {
    const int idx = tid + k * 256, e = idx >> 5, c = idx & 31;
    uint32_t b[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      b[2 * w] = fp8x2_to_bf16x2<false>((uint32_t)lat[k][w]);
      b[2 * w + 1] = fp8x2_to_bf16x2<true>((uint32_t)lat[k][w]);
    }
    uint16_t* dst = &s_k[e * kKStride + 16 * c];
    *reinterpret_cast<v4i*>(dst) = v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    *reinterpret_cast<v4i*>(dst + 8) = v4i{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
  }
#pragma unroll
  for (int k = 0; k < kCh / 32; ++k) {
    const int idx = tid + k * 256, e = idx >> 3, c = idx & 7;
    *reinterpret_cast<v4i*>(&s_k[e * kKStride + kLatent + 8 * c]) = rp[k];
  }
  if (tid < kCh) s_sc[tid] = scv;
  // copy mode: the codes, as gathered, into the per-slice value copy
  if (bc.z == 0 && !ent) {
#pragma unroll
    for (int k = 0; k < kCh / 8; ++k) {
      const int idx = tid + k * 256, e = idx >> 5, c = idx & 31;
      *reinterpret_cast<v4i*>(vc_t + ((int64_t)(c >> 2) * e_pad + e0 + e) * kSlice + 16 * (c & 3)) = lat[k];
    }
  }
  lds_sync();

  // scores of 16 heads x kCh entries (kCB 16-column blocks). The k-steps run
  // outermost, so consecutive matrix ops feed kCB independent accumulators
  // (a chain on one accumulator would wait out each op's latency), and the K
  // fragments are read twelve ahead of the matrix ops.
  v4f acc_l[kCB], acc_r[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc_l[cb] = acc_r[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  {
    constexpr int kAhead = 12, kNF = 18 * kCB;
    const uint16_t* kb = s_k + col * kKStride + grp * 8;
    auto kfrag = [&](int j) {
      return *reinterpret_cast<const v4i*>(kb + (j % kCB) * 16 * kKStride + (j / kCB) * 32);
    };
    v4i kf[kNF];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) kf[j] = kfrag(j);
    // one k-step per group; the scheduling fences keep the steps in order
#pragma unroll
    for (int s = 0; s < 18; ++s) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int j = s * kCB + cb;
        if (j + kAhead < kNF) kf[j + kAhead] = kfrag(j + kAhead);
        if (s < 16) acc_l[cb] = mfma_bf16(qa[s], kf[j], acc_l[cb]);
        else acc_r[cb] = mfma_bf16(qa[s], kf[j], acc_r[cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float sv[kCB][4];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int e = cb * 16 + col;
    const bool valid = s_es[e] >= 0;
    const float sc = s_sc[e];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[cb][r] = valid ? scale * fmaf(sc, acc_l[cb][r], acc_r[cb][r]) : -INFINITY;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = hbase + grp * 4 + r;
    float mr = sv[0][r];
#pragma unroll
    for (int cb = 1; cb < kCB; ++cb) mr = fmaxf(mr, sv[cb][r]);
    const float m = row16_max(mr);
    const bool dead = m == -INFINITY;
    float ps = 0.f;
    uint16_t* prow = pw + ((int64_t)t * H + h) * e_pad + e0;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const float pr = dead ? 0.f : __expf(sv[cb][r] - m);
      ps += pr;
      prow[cb * 16 + col] = f32_to_bf16(pr * s_sc[cb * 16 + col]);
    }
    const float l = row16_sum(ps);
    if (col == 0) stats[((int64_t)t * H + h) * n_chunks + chunk] = make_float2(m, l);
  }
}

// Phase B needs nothing of the query but phase A's outputs: the weights, the
// chunk statistics and the value slice of all e_pad entries (chunks past a
// list were written as zero / dead / zero). All of it is loaded in one round;
// the value slice goes to LDS row-major, and the P V products read their
// value operands from it with the transposing LDS load. kNC: chunk slots
// computed (the list's chunk count rounded up to even; extra slots are dead).
template <int kCh, int kNC, bool kOutF32, bool kGather>
__global__ void __launch_bounds__(256)
attn_pv_kernel(int H, const uint8_t* __restrict__ vcopy, const int32_t* __restrict__ ent,
               const uint8_t* __restrict__ c_lat, const uint8_t* __restrict__ r_lat,
               const uint16_t* __restrict__ pw,
               const float2* __restrict__ stats, int e_pad, void* __restrict__ out, int T,
               int nz, int g) {
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kNC * kCh * kVStride];
  __shared__ float s_f[64][kNC];
  const Coord bc = block_coord(kLatent / kSlice, nz, g);
  const int slice = bc.a, t = bc.t;
  if (t >= T) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int hb0 = bc.z * 64;
  const int n_chunks = e_pad / kCh;
  constexpr int kKS = kCh / 32;  // 32-entry k-steps per chunk

  // ---- first round of loads: statistics (first, so that the chunk factors
  // wait for them only), the value pieces (copy) or their slots (gather)
  // (16-B pieces j = tid + 256k: entry j / 4, dims 16 (j % 4) .. of the
  // slice), weights (A operands: 32-entry steps of this wave's 16 heads)
  v2f st[kNC];  // (m_c, l_c)
  {
    const float2* sp = stats + ((int64_t)t * H + hb0 + (tid & 63)) * n_chunks;
#pragma unroll
    for (int c = 0; c < kNC; ++c) st[c] = gload<v2f>((uint64_t)(sp + min(c, n_chunks - 1)));
  }
  asm volatile("" ::: "memory");  // keeps these loads ahead of the ones below
  constexpr int kVP = kNC * kCh * kSlice / 16 / 256;  // value pieces per thread
  const int nv = e_pad * (kSlice / 16);
  v4i vp[kVP];
  int32_t es[kVP];
  if (kGather) {
    const int32_t* ent_t = ent + (int64_t)t * e_pad;
#pragma unroll
    for (int k = 0; k < kVP; ++k) es[k] = gload<int32_t>((uint64_t)(ent_t + (min(tid + 256 * k, nv - 1) >> 2)));
  } else {
    const uint8_t* vsrc = vcopy + ((int64_t)t * (kLatent / kSlice) + slice) * e_pad * kSlice;
#pragma unroll
    for (int k = 0; k < kVP; ++k) vp[k] = gload<v4i>((uint64_t)(vsrc + 16 * min(tid + 256 * k, nv - 1)));
  }
  asm volatile("" ::: "memory");
  const uint64_t prow = (uint64_t)(pw + ((int64_t)t * H + hb0 + wave * 16 + col) * e_pad + grp * 8);
  v4i pa[kNC * kKS];
#pragma unroll
  for (int ks = 0; ks < kNC * kKS; ++ks) pa[ks] = gload<v4i>(prow + 2 * min(ks * 32, e_pad - 32));
  // gather, second round: the value pieces (a masked entry, or a piece past
  // e_pad, reads the zero row)
  if (kGather) {
#pragma unroll
    for (int k = 0; k < kVP; ++k) {
      const int j = tid + 256 * k;
      const Pick pk = pick_of(j < nv ? es[k] : -1);
      vp[k] = gload<v4i>(pick_base(pk, c_lat, r_lat, g_zero_row) + pk.slot * kLatent +
                         kSlice * slice + 16 * (j & 3));
    }
  }

  // chunk factors f_c = exp(m_c - M) / L of head hb0 + (tid & 63); every
  // wave computes them (a branch around the loads would let the compiler move
  // them behind the value loads) and wave 0 stores them
  {
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kNC; ++c)
      if (c < n_chunks) M = fmaxf(M, st[c].x);
    float Ls = 0.f;
#pragma unroll
    for (int c = 0; c < kNC; ++c)
      if (c < n_chunks && st[c].x != -INFINITY) Ls = fmaf(st[c].y, __expf(st[c].x - M), Ls);
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
#pragma unroll
    for (int c = 0; c < kNC; ++c) {
      const float f = (c < n_chunks && st[c].x != -INFINITY) ? __expf(st[c].x - M) * inv : 0.f;
      if (tid < 64) s_f[tid][c] = f;
    }
  }
  // values row-major [entry][64] in bf16 (exact); rows past e_pad are zeros
#pragma unroll
  for (int k = 0; k < kVP; ++k) {
    const int j = tid + 256 * k;
    uint32_t b[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = (kGather || j < nv) ? (uint32_t)vp[k][w] : 0u;
      b[2 * w] = fp8x2_to_bf16x2<false>(x);
      b[2 * w + 1] = fp8x2_to_bf16x2<true>(x);
    }
    uint16_t* dst = &s_v[(j >> 2) * kVStride + 16 * (j & 3)];
    *reinterpret_cast<v4i*>(dst) = v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    *reinterpret_cast<v4i*>(dst + 8) = v4i{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
  }
  lds_sync();

  // Every chunk slot is computed, straight-line: a chunk past the list has
  // f_c = 0 (and finite weights and values), and without a branch per chunk
  // the LDS reads and matrix ops of neighbouring chunks overlap. The value
  // operand (entries 8*grp..+7 of the step, dim col of block db) comes from
  // two transposing reads: lane 4a + b of a 16-lane group fetches entry
  // 8*grp + 4h + a, dims 4b..4b+3 of the block.
  const uint16_t* vb = s_v + (8 * grp + (col >> 2)) * kVStride + 4 * (col & 3);
  auto vfrag = [&](int c, int ks, int db) {
    const uint16_t* src = vb + (c * kCh + ks * 32) * kVStride + 16 * db;
    const v2i lo = __builtin_bit_cast(
        v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)src));
    const v2i hi = __builtin_bit_cast(
        v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                 (__attribute__((address_space(3))) v4s*)(src + 4 * kVStride)));
    return v4i{lo[0], lo[1], hi[0], hi[1]};
  };
  // Software pipeline over the chunks, one step per chunk: step c reads the
  // value fragments and factors of chunk c + 1, runs chunk c's products into
  // its own accumulators and folds chunk c - 1's (finished a step earlier)
  // into O, so no op waits on the one just issued. The scheduling fences keep
  // the steps in this order.
  v4f o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i vf[kNC][4 * kKS];
  float fc[kNC][4];
  v4f acc[kNC][4];
#pragma unroll
  for (int i = 0; i < 4 * kKS; ++i) vf[0][i] = vfrag(0, i >> 2, i & 3);
#pragma unroll
  for (int r = 0; r < 4; ++r) fc[0][r] = s_f[wave * 16 + grp * 4 + r][0];
#pragma unroll
  for (int c = 0; c <= kNC; ++c) {
    if (c + 1 < kNC) {
#pragma unroll
      for (int i = 0; i < 4 * kKS; ++i) vf[c + 1][i] = vfrag(c + 1, i >> 2, i & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) fc[c + 1][r] = s_f[wave * 16 + grp * 4 + r][c + 1];
    }
    if (c < kNC) {
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[c][db] = mfma_bf16(pa[c * kKS], vf[c][db], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < kKS; ++ks)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[c][db] = mfma_bf16(pa[c * kKS + ks], vf[c][4 * ks + db], acc[c][db]);
    }
    if (c > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][r] = fmaf(fc[c - 1][r], acc[c - 1][db][r], o[db][r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t ob = ((int64_t)t * H + hb0 + wave * 16 + grp * 4 + r) * kLatent + slice * kSlice + col;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      if (kOutF32) reinterpret_cast<float*>(out)[ob + db * 16] = o[db][r];
      else reinterpret_cast<uint16_t*>(out)[ob + db * 16] = f32_to_bf16(o[db][r]);
    }
  }
}

// The two-phase path for up to 64 (query, 64-head block) units: at 128 (32
// sequences x 4 query tokens at 128K) the split kernel with two splits and the
// combine took 50 us against 58 us for the two phases.
bool use_two_phase(int T, int H, int max_entries) {
  return H % 64 == 0 && T * (H / 64) <= 64 && max_entries <= kTwoPhaseMaxE && max_entries > 0;
}

// Entries per phase-A workgroup: 64, or 96 when 64-entry chunks make more
// workgroups than the GPU has CUs and 96-entry ones do not. Phase A's
// workgroups run one round, and a CU that holds two of them takes about 1.5x
// as long as one that holds one (32 queries x 64 heads x 640 entries: 320
// workgroups, 11.6 us; the same list for 24 queries, 240 workgroups, 7.7
// us), so the kernel lasts as long as its doubly loaded CUs. The grid's size
// decides: block_coord spreads it evenly over the eight XCDs of 32 CUs.
int two_phase_chunk(int T, int H, int max_entries) {
  const int nz = H / 64;
  const unsigned g64 = xcd_grid((max_entries + kChunk - 1) / kChunk, nz, T).x;
  const unsigned gw = xcd_grid((max_entries + kChunkWide - 1) / kChunkWide, nz, T).x;
  return (g64 > (unsigned)kAttnCUs && gw <= (unsigned)kAttnCUs) ? kChunkWide : kChunk;
}

// Workspace of the two-phase path: P' [T][H][e_pad] bf16, then the chunk
// statistics [T][H][e_pad/ch] float2 (ch = two_phase_chunk), then phase B's
// value source: the entries' slot codes [T][e_pad] int32 (slot * 2 + pool, -1 when masked) in
// gather mode, the value copy [T][8][e_pad][64] (FP8 codes, one block per
// 64-dim slice) in copy mode.
struct TwoPhaseWs {
  size_t pw, stats, src, total;
  bool gather;
};
TwoPhaseWs two_phase_ws(int64_t T, int H, int e_pad, int ch) {
  TwoPhaseWs w;
  w.pw = 0;
  w.stats = ((size_t)T * H * e_pad * 2 + 255) / 256 * 256;
  w.src = w.stats + ((size_t)T * H * (e_pad / ch) * sizeof(float2) + 255) / 256 * 256;
  const size_t copy = (size_t)T * e_pad * kLatent;
  w.gather = copy >= kGatherMinCopy;
  w.total = w.src + (w.gather ? (size_t)T * e_pad * sizeof(int32_t) : copy);
  return w;
}

// fp32 pools and queries (small configurations). A query's entry list is cut
// into 16-entry chunks; a workgroup stages one chunk (576 floats per entry,
// read as coalesced 16-byte loads) and the query rows of up to 16 heads in
// LDS, scores the chunk, takes each head's max and exponent sum over it and
// the partial P V. attn_f32_combine_kernel merges the chunks of a (query,
// head) exactly (each partial rescaled by exp(m_c - M)); with a single chunk
// the first kernel writes the output itself. An empty list gives zeros.
constexpr int kF32Chunk = 16;  // entries per workgroup (16: the tiny decode's 640 entries make 40 workgroups)
constexpr int kF32Heads = 16;  // heads per workgroup
constexpr int kF32Row = kKvDim + 4;  // LDS row stride (floats)

__global__ void __launch_bounds__(256)
attn_f32_chunk_kernel(const float* __restrict__ q, int H, const int32_t* __restrict__ q_seq,
                      const int32_t* __restrict__ q_pos, bool hca,
                      const int32_t* __restrict__ phys_idx, int k_sel, int ratio, csa_kv_pool comp,
                      const int32_t* __restrict__ comp_pt, int comp_pt_stride, csa_kv_pool raw,
                      const int32_t* __restrict__ raw_pt, int raw_pt_stride, int window,
                      float scale, float* __restrict__ out, float* __restrict__ part, int nchunk) {
  __shared__ __attribute__((aligned(16))) float s_kv[kF32Chunk * kF32Row];
  __shared__ __attribute__((aligned(16))) float s_q[kF32Heads * kF32Row];
  __shared__ float s_p[kF32Chunk][kF32Heads + 1];
  __shared__ float s_m[kF32Heads], s_l[kF32Heads];
  __shared__ int64_t s_slot[kF32Chunk];
  __shared__ int s_pool[kF32Chunk];
  const int c = blockIdx.x, t = blockIdx.z;
  const int h0 = blockIdx.y * kF32Heads;
  const int nh = min(kF32Heads, H - h0);
  const int tid = threadIdx.x;
  const int seq = q_seq[t], p = q_pos[t];
  const EntryList L = entry_list(p, k_sel, hca, ratio, window);
  const int total = L.n1 + L.n2;
  const int e0 = c * kF32Chunk;
  if (tid < kF32Chunk) {
    int pool = 0;
    int64_t slot = -1;
    if (e0 + tid < total)
      slot = entry_slot(e0 + tid, L, t, seq, hca, phys_idx, k_sel, comp_pt, comp_pt_stride,
                        comp.page_size, raw_pt, raw_pt_stride, raw.page_size, pool);
    s_slot[tid] = slot;
    s_pool[tid] = pool;
  }
  // query rows of this workgroup's heads (rows past nh are zero): all of a
  // thread's loads are issued before any is stored, so they overlap
  constexpr int kQv = kF32Heads * (kKvDim / 4) / 256;  // float4 per thread
  {
    float4 v[kQv];
#pragma unroll
    for (int r = 0; r < kQv; ++r) {
      const int i = tid + 256 * r, h = i / (kKvDim / 4), f = i % (kKvDim / 4);
      v[r] = h < nh ? reinterpret_cast<const float4*>(q + ((int64_t)t * H + h0 + h) * kKvDim)[f]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < kQv; ++r) {
      const int i = tid + 256 * r, h = i / (kKvDim / 4), f = i % (kKvDim / 4);
      *reinterpret_cast<float4*>(&s_q[h * kF32Row + 4 * f]) = v[r];
    }
  }
  __syncthreads();
  // the chunk's entries: 128 float4 of latent and 16 of RoPE dims each, all
  // loads in flight at once
  constexpr int kKv = kF32Chunk * (kKvDim / 4) / 256;  // float4 per thread
  {
    float4 v[kKv];
#pragma unroll
    for (int r = 0; r < kKv; ++r) {
      const int i = tid + 256 * r, e = i / (kKvDim / 4), f = i % (kKvDim / 4);
      const int64_t slot = s_slot[e];
      const csa_kv_pool& P = s_pool[e] ? raw : comp;
      const int64_t sl = slot >= 0 ? slot : 0;
      const float4* src = f < kLatent / 4
                              ? reinterpret_cast<const float4*>(P.latent) + sl * (kLatent / 4) + f
                              : reinterpret_cast<const float4*>(P.rope) + sl * (kRope / 4) + f - kLatent / 4;
      v[r] = slot >= 0 ? *src : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < kKv; ++r) {
      const int i = tid + 256 * r, e = i / (kKvDim / 4), f = i % (kKvDim / 4);
      *reinterpret_cast<float4*>(&s_kv[e * kF32Row + 4 * f]) = v[r];
    }
  }
  __syncthreads();
  static_assert(kF32Chunk == 16 && kF32Heads == 16, "the lane layouts below");
  {  // scores: lane (eb, hb, kp) forms the 4 x 4 block of entries 4 eb.. and
     // heads 4 hb.. over dims [36 kp, 36 kp + 36); the sixteen dim parts are
     // summed across a 16-lane row (kp = lane % 16)
    const int kp = tid & 15, hb = (tid >> 4) & 3, eb = tid >> 6;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 3
    for (int k = kp * 36; k < kp * 36 + 36; k += 4) {
      float4 kv[4], qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kv[i] = *reinterpret_cast<const float4*>(&s_kv[(eb * 4 + i) * kF32Row + k]);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[j] = *reinterpret_cast<const float4*>(&s_q[(hb * 4 + j) * kF32Row + k]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = fmaf(qv[j].x, kv[i].x, fmaf(qv[j].y, kv[i].y,
                      fmaf(qv[j].z, kv[i].z, fmaf(qv[j].w, kv[i].w, acc[i][j]))));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = acc[i][j];
        v += lane_xor<1>(v);
        v += lane_xor<2>(v);
        v += lane_xor<4>(v);
        v += lane_xor<8>(v);
        acc[i][j] = v;
      }
    // lane kp writes entry / head (i, j) with 4 i + j == kp
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * i + j == kp) {
          const int e = eb * 4 + i;
          s_p[e][hb * 4 + j] = s_slot[e] >= 0 ? acc[i][j] * scale : -INFINITY;
        }
  }
  __syncthreads();
  {  // the chunk's max and exponent sum per head: a 16-lane row per head,
     // one entry per lane
    const int h = tid >> 4, r = tid & 15;
    const float s0 = s_p[r][h];
    const float m = row16_max(s0);
    const float p0 = s0 == -INFINITY ? 0.f : expf(s0 - m);
    const float l = row16_sum(p0);
    s_p[r][h] = p0;
    if (r == 0) {
      s_m[h] = m;
      s_l[h] = l;
    }
  }
  __syncthreads();
  // P V over the chunk: this thread's value dims 2 tid, 2 tid + 1, every head
  float acc[kF32Heads][2];
#pragma unroll
  for (int h = 0; h < kF32Heads; ++h) acc[h][0] = acc[h][1] = 0.f;
  for (int e = 0; e < kF32Chunk; ++e) {
    const float2 v = *reinterpret_cast<const float2*>(&s_kv[e * kF32Row + 2 * tid]);
#pragma unroll
    for (int h = 0; h < kF32Heads; ++h) {
      const float pe = s_p[e][h];
      acc[h][0] = fmaf(pe, v.x, acc[h][0]);
      acc[h][1] = fmaf(pe, v.y, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < kF32Heads; ++h) {
    if (h >= nh) continue;
    if (nchunk == 1) {
      const float l = s_l[h];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      *reinterpret_cast<float2*>(out + ((int64_t)t * H + h0 + h) * kLatent + 2 * tid) =
          make_float2(acc[h][0] * inv, acc[h][1] * inv);
    } else {
      float* dst = part + (((int64_t)t * nchunk + c) * H + h0 + h) * (kLatent + 2);
      if (tid == 0) {
        dst[0] = s_m[h];
        dst[1] = s_l[h];
      }
      dst[2 + 2 * tid] = acc[h][0];
      dst[3 + 2 * tid] = acc[h][1];
    }
  }
}

// Merge of the chunks of one (query, head): O = sum_c e^(m_c - M) O_c /
// sum_c e^(m_c - M) l_c over the chunks with entries (l_c > 0). The chunks'
// (m, l) come in with one parallel load into LDS; each thread then reads its
// two value dims of every chunk with independent loads.
constexpr int kF32MaxChunks = 2048;  // chunks merged by one workgroup (32768 entries)
__global__ void __launch_bounds__(256)
attn_f32_combine_kernel(const float* __restrict__ part, int H, int nchunk, float* __restrict__ out) {
  __shared__ float s_f[kF32MaxChunks];
  __shared__ float s_red[8];
  const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int64_t cs = (int64_t)H * (kLatent + 2);
  const float* base = part + ((int64_t)t * nchunk * H + h) * (kLatent + 2);
  float mx = -INFINITY;
  for (int c = tid; c < nchunk; c += 256) {
    const float2 ml = *reinterpret_cast<const float2*>(base + c * cs);
    s_f[c] = ml.y > 0.f ? ml.x : -INFINITY;
    mx = fmaxf(mx, s_f[c]);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  float ls = 0.f;
  for (int c = tid; c < nchunk; c += 256) {
    const float l = base[c * cs + 1];
    const float f = s_f[c] == -INFINITY ? 0.f : expf(s_f[c] - M);
    s_f[c] = f;
    ls = fmaf(l, f, ls);
  }
  ls = wave_sum(ls);
  __syncthreads();
  if ((tid & 63) == 0) s_red[4 + (tid >> 6)] = ls;
  __syncthreads();
  const float L = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll 8
  for (int c = 0; c < nchunk; ++c) {
    const float2 v = *reinterpret_cast<const float2*>(base + c * cs + 2 + 2 * tid);
    const float f = s_f[c];
    o0 = fmaf(f, v.x, o0);
    o1 = fmaf(f, v.y, o1);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float2*>(out + ((int64_t)t * H + h) * kLatent + 2 * tid) =
      make_float2(o0 * inv, o1 * inv);
}

int pick_splits(int T, int H, int max_entries) {
  // About one workgroup per CU (256), each split at least two tiles long and
  // at most kMaxSplit entries.
  const int hblocks = H >= 64 ? H / 64 : 1;
  const int max_split = (max_entries + 2 * kTile - 1) / (2 * kTile);
  int s = (256 + T * hblocks - 1) / (T * hblocks);
  if (s > max_split) s = max_split;
  const int min_split = (max_entries + kMaxSplit - 1) / kMaxSplit;
  if (s < min_split) s = min_split;
  return s < 1 ? 1 : s;
}

// How the split kernel divides the entry lists. Uniform: nsplit pieces of
// split_len per query. Balanced (few queries of one head block, e.g. HCA over
// ragged lengths, where a uniform cut leaves the longest list's pieces
// setting the kernel's span): `slots` workgroups shared out by list length
// inside the kernel, at least 256 and enough for pieces of at most kMaxSplit.
struct SplitPlan {
  bool balanced;
  int nsplit, split_len, slots;
  size_t part_bytes, qsplit_bytes;
};
SplitPlan split_plan(int T, int H, int max_entries) {
  SplitPlan p{};
  p.nsplit = pick_splits(T, H, max_entries);
  const int nw = H >= 64 ? 4 : H / 16;
  const int nz = H / (16 * nw);
  p.balanced = p.nsplit > 1 && T <= 64 && nz == 1;
  if (p.balanced) {
    p.slots = std::max(256, T * ((max_entries + kMaxSplit - 1) / kMaxSplit) + T);
    p.part_bytes = (size_t)p.slots * H * (kLatent + 2) * sizeof(float);
    p.qsplit_bytes = (size_t)T * sizeof(int2);
  } else {
    p.slots = T * p.nsplit;
    p.split_len = ((max_entries + p.nsplit - 1) / p.nsplit + kTile - 1) / kTile * kTile;
    p.part_bytes = p.nsplit > 1 ? (size_t)T * p.nsplit * H * (kLatent + 2) * sizeof(float) : 0;
  }
  return p;
}

}  // namespace

size_t attention_f32_ws_bytes(int64_t T, int64_t max_entries, int H) {
  const int64_t nchunk = (max_entries + kF32Chunk - 1) / kF32Chunk;
  return nchunk > 1 ? (size_t)T * nchunk * H * (kLatent + 2) * sizeof(float) : 0;
}

size_t attention_ws_bytes(int64_t T, int64_t max_entries, int H) {
  if (use_two_phase((int)T, H, (int)max_entries)) {
    const int ch = two_phase_chunk((int)T, H, (int)max_entries);
    return two_phase_ws(T, H, (int)((max_entries + ch - 1) / ch * ch), ch).total;
  }
  const SplitPlan p = split_plan((int)T, H, (int)max_entries);
  return p.part_bytes + p.qsplit_bytes;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int max_entries = a.max_comp + a.window;
  if (a.comp.fmt == CSA_F32) {
    const int nchunk = std::max(1, (max_entries + kF32Chunk - 1) / kF32Chunk);
    if (nchunk > kF32MaxChunks) return hipErrorInvalidValue;
    float* part = (float*)a.ws;
    hipLaunchKernelGGL(attn_f32_chunk_kernel, dim3(nchunk, (a.H + kF32Heads - 1) / kF32Heads, a.T),
                       dim3(256), 0, s, (const float*)a.q, a.H, a.q_seq, a.q_pos, a.hca, a.phys_idx,
                       a.k_sel, a.ratio, a.comp, a.comp_pt, a.comp_pt_stride, a.raw, a.raw_pt,
                       a.raw_pt_stride, a.window, a.scale, (float*)a.out, part, nchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nchunk == 1) return e;
    hipLaunchKernelGGL(attn_f32_combine_kernel, dim3(a.H, a.T), dim3(256), 0, s, part, a.H, nchunk,
                       (float*)a.out);
    return hipGetLastError();
  }
  if (use_two_phase(a.T, a.H, max_entries)) {
    const int ch = two_phase_chunk(a.T, a.H, max_entries);
    const int e_pad = (max_entries + ch - 1) / ch * ch;
    const TwoPhaseWs w = two_phase_ws(a.T, a.H, e_pad, ch);
    uint16_t* pw = (uint16_t*)((char*)a.ws + w.pw);
    float2* st = (float2*)((char*)a.ws + w.stats);
    uint8_t* vc = w.gather ? nullptr : (uint8_t*)a.ws + w.src;
    int32_t* ent = w.gather ? (int32_t*)((char*)a.ws + w.src) : nullptr;
    const int nz = a.H / 64;
    const int g = xcd_group(a.T);
#define CSA_SCORES(CH)                                                                        \
  hipLaunchKernelGGL((attn_scores_kernel<CH>), xcd_grid(e_pad / CH, nz, a.T), dim3(256), 0, s,     \
                     (const uint16_t*)a.q, a.H, a.q_seq, a.q_pos, a.hca, a.phys_idx, a.k_sel,      \
                     a.ratio, (const uint8_t*)a.comp.latent, a.comp.latent_scale,                \
                     (const uint16_t*)a.comp.rope, a.comp.page_size, a.comp_pt, a.comp_pt_stride, \
                     (const uint8_t*)a.raw.latent, a.raw.latent_scale,                            \
                     (const uint16_t*)a.raw.rope, a.raw.page_size, a.raw_pt, a.raw_pt_stride,     \
                     a.window, a.scale, pw, st, vc, ent, e_pad, a.T, nz, g)
    if (ch == kChunkWide) CSA_SCORES(kChunkWide);
    else CSA_SCORES(kChunk);
#undef CSA_SCORES
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define CSA_PV(CH, NC, FO, GA)                                                                  \
  hipLaunchKernelGGL((attn_pv_kernel<CH, NC, FO, GA>), xcd_grid(kLatent / kSlice, nz, a.T), dim3(256), \
                     0, s, a.H, vc, ent, (const uint8_t*)a.comp.latent, (const uint8_t*)a.raw.latent, \
                     pw, st, e_pad, a.out, a.T, nz, g)
#define CSA_PV_NC(CH, NC)                               \
  case NC:                                              \
    if (a.out_fmt == CSA_F32) {                         \
      if (w.gather) CSA_PV(CH, NC, true, true);         \
      else CSA_PV(CH, NC, true, false);                 \
    } else {                                            \
      if (w.gather) CSA_PV(CH, NC, false, true);        \
      else CSA_PV(CH, NC, false, false);                \
    }                                                   \
    break;
    // chunk slots: the list's chunks rounded up to even (the extra one is dead)
    const int nc = (e_pad / ch + 1) / 2 * 2;
    if (ch == kChunkWide) {
      switch (nc) {
        CSA_PV_NC(kChunkWide, 2)
        CSA_PV_NC(kChunkWide, 4)
        CSA_PV_NC(kChunkWide, 6)
        CSA_PV_NC(kChunkWide, 8)
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (nc) {
        CSA_PV_NC(kChunk, 2)
        CSA_PV_NC(kChunk, 4)
        CSA_PV_NC(kChunk, 6)
        CSA_PV_NC(kChunk, 8)
        CSA_PV_NC(kChunk, 10)
        CSA_PV_NC(kChunk, 12)
        default: return hipErrorInvalidValue;
      }
    }
#undef CSA_PV_NC
#undef CSA_PV
    return hipGetLastError();
  }
  const SplitPlan sp = split_plan(a.T, a.H, max_entries);
  const int nsplit = sp.balanced ? sp.slots : sp.nsplit;  // the kernels' nsplit argument
  const int split_len = sp.split_len;
  const bool f32o = a.out_fmt == CSA_F32;
  float* part = sp.nsplit > 1 ? (float*)a.ws : nullptr;
  int2* qsplit = sp.balanced ? (int2*)((char*)a.ws + sp.part_bytes) : nullptr;
  const int nw = a.H >= 64 ? 4 : a.H / 16;  // pairs of waves per workgroup (16 heads each)
  const int nz = a.H / (16 * nw);
  const int g = xcd_group(a.T);
  const dim3 grid = sp.balanced ? dim3((unsigned)sp.slots) : xcd_grid(nsplit, nz, a.T);
#define CSA_ATTN(NW, FO)                                                                      \
  hipLaunchKernelGGL((attn_mfma_kernel<NW, FO>), grid, dim3(NW * 128), 0, s,                 \
                     (const uint16_t*)a.q, a.H, a.q_seq, a.q_pos, a.hca, a.phys_idx, a.k_sel,   \
                     a.ratio, (const uint8_t*)a.comp.latent, a.comp.latent_scale,             \
                     (const uint16_t*)a.comp.rope, a.comp.page_size, a.comp_pt,              \
                     a.comp_pt_stride, (const uint8_t*)a.raw.latent, a.raw.latent_scale,      \
                     (const uint16_t*)a.raw.rope, a.raw.page_size, a.raw_pt, a.raw_pt_stride, \
                     a.window, a.scale, a.out, part, split_len, nsplit, a.T, nz, g, qsplit)
  if (nw == 4) { if (f32o) CSA_ATTN(4, true); else CSA_ATTN(4, false); }
  else if (nw == 2) { if (f32o) CSA_ATTN(2, true); else CSA_ATTN(2, false); }
  else { if (f32o) CSA_ATTN(1, true); else CSA_ATTN(1, false); }
#undef CSA_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.nsplit == 1) return e;
  if (sp.balanced) {
    if (f32o)
      hipLaunchKernelGGL(attn_combine_slots_kernel<true>, xcd_grid(a.H, 1, a.T), dim3(256), 0, s,
                         part, a.T, a.H, nsplit, a.out, g, qsplit);
    else
      hipLaunchKernelGGL(attn_combine_slots_kernel<false>, xcd_grid(a.H, 1, a.T), dim3(256), 0, s,
                         part, a.T, a.H, nsplit, a.out, g, qsplit);
  } else if (f32o)
    hipLaunchKernelGGL(attn_combine_kernel<true>, xcd_grid(a.H / 4, 1, a.T), dim3(256), 0, s,
                       part, a.T, a.H, nsplit, a.out, g, qsplit);
  else
    hipLaunchKernelGGL(attn_combine_kernel<false>, xcd_grid(a.H / 4, 1, a.T), dim3(256), 0, s,
                       part, a.T, a.H, nsplit, a.out, g, qsplit);
  return hipGetLastError();
}

}  // namespace csa
