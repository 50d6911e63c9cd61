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
// A workgroup owns one query and a contiguous range of its entry list; wave w
// owns heads 16w..16w+15. Entries are gathered 32 at a time into LDS (codes
// row-major for S, bf16 V^T for the value product), then every wave runs its
// heads against the shared tile with an online softmax. Long entry lists are
// split over several workgroups whose partial (max, sum, O) are merged by a
// second kernel.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {
namespace {

constexpr int kTile = 32;             // entries per LDS tile
constexpr int kLatStride = 528;       // bytes per row of the fp8 code tile
constexpr int kVtStride = kTile + 8;  // bf16 elements per row of V^T
constexpr int kRopeStride = 72;       // bf16 elements per row of the RoPE tile
constexpr int kPStride = kTile + 8;   // bf16 elements per row of P

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

template <int kNW, bool kOutF32>
__global__ void __launch_bounds__(kNW * 64)
attn_mfma_kernel(const uint16_t* __restrict__ q, int H, const int32_t* __restrict__ q_seq,
                 const int32_t* __restrict__ q_pos, bool hca, const int32_t* __restrict__ phys_idx,
                 int k_sel, int ratio, csa_kv_pool comp, const int32_t* __restrict__ comp_pt,
                 int comp_pt_stride, csa_kv_pool raw, const int32_t* __restrict__ raw_pt,
                 int raw_pt_stride, int window, float scale, void* __restrict__ out,
                 float* __restrict__ part, int split_len, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint8_t s_lat[kTile * kLatStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[kLatent * kVtStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_rope[kTile * kRopeStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_p[kNW][16 * kPStride];
  __shared__ float s_scale[kTile];
  __shared__ int s_valid[kTile];

  const int t = blockIdx.y;
  const int split = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int seq = q_seq[t];
  const int p = q_pos[t];
  const EntryList L = entry_list(p, k_sel, hca, ratio, window);
  const int total = L.n1 + L.n2;
  const int e_begin = split * split_len;
  const int e_end = min(total, e_begin + split_len);

  // Heads of this wave: hbase + 16*wave .. +15 (grid.z splits H in blocks of 16*kNW).
  const int hbase = blockIdx.z * kNW * 16 + wave * 16;
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

  float m[4], l[4];
  v4f o[32];
#pragma unroll
  for (int r = 0; r < 4; ++r) { m[r] = -INFINITY; l[r] = 0.f; }
#pragma unroll
  for (int n = 0; n < 32; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nthreads = kNW * 64;
  for (int tile0 = e_begin; tile0 < e_end; tile0 += kTile) {
    // ---- gather the tile into LDS
    if (threadIdx.x < kTile) {
      const int i = tile0 + threadIdx.x;
      int pool = 0;
      int64_t slot = -1;
      if (i < e_end)
        slot = entry_slot(i, L, t, seq, hca, phys_idx, k_sel, comp_pt, comp_pt_stride,
                          comp.page_size, raw_pt, raw_pt_stride, raw.page_size, pool);
      s_valid[threadIdx.x] = slot >= 0 ? (int)(slot * 2 + pool) + 1 : 0;  // packed, 0 = masked
    }
    __syncthreads();
    // latent codes: 32 entries x 32 chunks of 16 B
    for (int c = threadIdx.x; c < kTile * 32; c += nthreads) {
      const int e = c & (kTile - 1);
      const int ch = c >> 5;
      const int v = s_valid[e];
      uint4 x = make_uint4(0, 0, 0, 0);
      if (v) {
        const int64_t slot = (int64_t)((v - 1) >> 1);
        const uint8_t* base = (const uint8_t*)(((v - 1) & 1) ? raw.latent : comp.latent);
        x = *reinterpret_cast<const uint4*>(base + slot * kLatent + ch * 16);
      }
      *reinterpret_cast<uint4*>(s_lat + e * kLatStride + ch * 16) = x;
      const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t code = (w4[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        s_vt[(ch * 16 + i) * kVtStride + e] = (uint16_t)e4m3_to_bf16(code);
      }
    }
    // RoPE dims: 32 entries x 8 chunks of 16 B; scales
    for (int c = threadIdx.x; c < kTile * 8; c += nthreads) {
      const int e = c & (kTile - 1);
      const int ch = c >> 5;
      const int v = s_valid[e];
      uint4 x = make_uint4(0, 0, 0, 0);
      if (v) {
        const int64_t slot = (int64_t)((v - 1) >> 1);
        const uint16_t* base = (const uint16_t*)(((v - 1) & 1) ? raw.rope : comp.rope);
        x = *reinterpret_cast<const uint4*>(base + slot * kRope + ch * 8);
      }
      *reinterpret_cast<uint4*>(s_rope + e * kRopeStride + ch * 8) = x;
    }
    if (threadIdx.x < kTile) {
      const int v = s_valid[threadIdx.x];
      float sc = 0.f;
      if (v) {
        const int64_t slot = (int64_t)((v - 1) >> 1);
        sc = (((v - 1) & 1) ? raw.latent_scale : comp.latent_scale)[slot];
      }
      s_scale[threadIdx.x] = sc;
    }
    __syncthreads();

    // ---- S = Q K^T for 16 heads x 32 entries (two 16-column blocks)
    float sv[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int e = cb * 16 + col;
      v4f acc_l = {0.f, 0.f, 0.f, 0.f}, acc_r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(s_lat + e * kLatStride + s * 32 + grp * 8);
        v4i bk;
        bk[0] = (int)(e4m3_to_bf16(c8.x & 0xFF) | (e4m3_to_bf16((c8.x >> 8) & 0xFF) << 16));
        bk[1] = (int)(e4m3_to_bf16((c8.x >> 16) & 0xFF) | (e4m3_to_bf16(c8.x >> 24) << 16));
        bk[2] = (int)(e4m3_to_bf16(c8.y & 0xFF) | (e4m3_to_bf16((c8.y >> 8) & 0xFF) << 16));
        bk[3] = (int)(e4m3_to_bf16((c8.y >> 16) & 0xFF) | (e4m3_to_bf16(c8.y >> 24) << 16));
        acc_l = mfma_bf16(qa[s], bk, acc_l);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint4 r8 = *reinterpret_cast<const uint4*>(s_rope + e * kRopeStride + s * 32 + grp * 8);
        acc_r = mfma_bf16(qa[16 + s], v4i{(int)r8.x, (int)r8.y, (int)r8.z, (int)r8.w}, acc_r);
      }
      const bool valid = s_valid[e] != 0;
      const float sc = s_scale[e];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sv[cb][r] = valid ? scale * fmaf(sc, acc_l[r], acc_r[r]) : -INFINITY;
    }
    // ---- online softmax over the tile (rows = heads 4*grp + r)
    float corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mt = fmaxf(sv[0][r], sv[1][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 1, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 2, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 4, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 8, 64));
      const float mn = fmaxf(m[r], mt);
      const bool dead = mn == -INFINITY;
      corr[r] = dead ? 1.f : __expf(m[r] - mn);
      const float p0 = dead ? 0.f : __expf(sv[0][r] - mn);
      const float p1 = dead ? 0.f : __expf(sv[1][r] - mn);
      float ps = p0 + p1;
      ps += __shfl_xor(ps, 1, 64);
      ps += __shfl_xor(ps, 2, 64);
      ps += __shfl_xor(ps, 4, 64);
      ps += __shfl_xor(ps, 8, 64);
      l[r] = l[r] * corr[r] + ps;
      m[r] = mn;
      // P' = p * (value dequant scale), bf16, stored row-major [head][entry]
      uint16_t* prow = &s_p[wave][(grp * 4 + r) * kPStride];
      prow[col] = f32_to_bf16(p0 * s_scale[col]);
      prow[16 + col] = f32_to_bf16(p1 * s_scale[16 + col]);
    }
#pragma unroll
    for (int n = 0; n < 32; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[n][r] *= corr[r];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): P stores visible to the wave
    __builtin_amdgcn_wave_barrier();
    // ---- O += P V: A = P (head col, entries grp*8..+7), B = V^T rows
    const uint4 pa8 = *reinterpret_cast<const uint4*>(&s_p[wave][col * kPStride + grp * 8]);
    const v4i pa = v4i{(int)pa8.x, (int)pa8.y, (int)pa8.z, (int)pa8.w};
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      const uint4 v8 = *reinterpret_cast<const uint4*>(&s_vt[(n * 16 + col) * kVtStride + grp * 8]);
      o[n] = mfma_bf16(pa, v4i{(int)v8.x, (int)v8.y, (int)v8.z, (int)v8.w}, o[n]);
    }
    __syncthreads();
  }

  const int h0 = hbase + grp * 4;
  if (nsplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
      const int64_t obase = ((int64_t)t * H + h0 + r) * kLatent + col;
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        const float v = o[n][r] * inv;
        if (kOutF32) reinterpret_cast<float*>(out)[obase + n * 16] = v;
        else reinterpret_cast<uint16_t*>(out)[obase + n * 16] = f32_to_bf16(v);
      }
    }
  } else {
    // partials: [T][nsplit][H][512] O, then [T][nsplit][H] m and l
    const int64_t ph = ((int64_t)t * nsplit + split) * H;
    float* po = part;
    float* pm = part + (int64_t)gridDim.y * nsplit * H * kLatent;
    float* pl = pm + (int64_t)gridDim.y * nsplit * H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t obase = (ph + h0 + r) * kLatent + col;
#pragma unroll
      for (int n = 0; n < 32; ++n) po[obase + n * 16] = o[n][r];
      if (col == 0) {
        pm[ph + h0 + r] = m[r];
        pl[ph + h0 + r] = l[r];
      }
    }
  }
}

template <bool kOutF32>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part, int T, int H, int nsplit,
                    void* __restrict__ out) {
  const int t = blockIdx.y;
  const int h = blockIdx.x;
  const float* pm = part + (int64_t)T * nsplit * H * kLatent;
  const float* pl = pm + (int64_t)T * nsplit * H;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pm[((int64_t)t * nsplit + s) * H + h]);
  float Lsum = 0.f;
  float acc0 = 0.f, acc1 = 0.f;
  const int d0 = threadIdx.x, d1 = threadIdx.x + 256;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t idx = ((int64_t)t * nsplit + s) * H + h;
    const float ms = pm[idx];
    if (ms == -INFINITY) continue;
    const float f = __expf(ms - M);
    Lsum = fmaf(pl[idx], f, Lsum);
    acc0 = fmaf(part[idx * kLatent + d0], f, acc0);
    acc1 = fmaf(part[idx * kLatent + d1], f, acc1);
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int64_t ob = ((int64_t)t * H + h) * kLatent;
  if (kOutF32) {
    reinterpret_cast<float*>(out)[ob + d0] = acc0 * inv;
    reinterpret_cast<float*>(out)[ob + d1] = acc1 * inv;
  } else {
    reinterpret_cast<uint16_t*>(out)[ob + d0] = f32_to_bf16(acc0 * inv);
    reinterpret_cast<uint16_t*>(out)[ob + d1] = f32_to_bf16(acc1 * inv);
  }
}

// fp32 pools and queries (small configurations): one workgroup per (query,
// head); scores in LDS, exact two-pass softmax, then the value sum.
__global__ void __launch_bounds__(256)
attn_f32_kernel(const float* __restrict__ q, int H, const int32_t* __restrict__ q_seq,
                const int32_t* __restrict__ q_pos, bool hca, const int32_t* __restrict__ phys_idx,
                int k_sel, int ratio, csa_kv_pool comp, const int32_t* __restrict__ comp_pt,
                int comp_pt_stride, csa_kv_pool raw, const int32_t* __restrict__ raw_pt,
                int raw_pt_stride, int window, float scale, float* __restrict__ out) {
  extern __shared__ float sh[];  // q[576], then scores[total], then red[8]
  const int t = blockIdx.y, h = blockIdx.x;
  const int seq = q_seq[t], p = q_pos[t];
  const EntryList L = entry_list(p, k_sel, hca, ratio, window);
  const int total = L.n1 + L.n2;
  float* sq = sh;
  float* ss = sh + kKvDim;
  float* red = ss + total;
  for (int i = threadIdx.x; i < kKvDim; i += blockDim.x) sq[i] = q[((int64_t)t * H + h) * kKvDim + i];
  __syncthreads();
  float lmax = -INFINITY;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    int pool;
    const int64_t slot = entry_slot(i, L, t, seq, hca, phys_idx, k_sel, comp_pt, comp_pt_stride,
                                    comp.page_size, raw_pt, raw_pt_stride, raw.page_size, pool);
    float s = -INFINITY;
    if (slot >= 0) {
      const csa_kv_pool& P = pool ? raw : comp;
      const float* lat = (const float*)P.latent + slot * kLatent;
      const float* rp = (const float*)P.rope + slot * kRope;
      float d = 0.f;
      for (int k = 0; k < kLatent; ++k) d = fmaf(sq[k], lat[k], d);
      for (int k = 0; k < kRope; ++k) d = fmaf(sq[kLatent + k], rp[k], d);
      s = d * scale;
    }
    ss[i] = s;
    lmax = fmaxf(lmax, s);
  }
  lmax = wave_max(lmax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lmax;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float lsum = 0.f;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const float e = ss[i] == -INFINITY ? 0.f : expf(ss[i] - M);
    ss[i] = e;
    lsum += e;
  }
  lsum = wave_sum(lsum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lsum;
  __syncthreads();
  float S = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) S += red[i];
  const float inv = 1.f / S;
  for (int d = threadIdx.x; d < kLatent; d += blockDim.x) {
    float acc = 0.f;
    for (int i = 0; i < total; ++i) {
      const float pe = ss[i];
      if (pe == 0.f) continue;
      int pool;
      const int64_t slot = entry_slot(i, L, t, seq, hca, phys_idx, k_sel, comp_pt, comp_pt_stride,
                                      comp.page_size, raw_pt, raw_pt_stride, raw.page_size, pool);
      const csa_kv_pool& P = pool ? raw : comp;
      acc = fmaf(pe, ((const float*)P.latent)[slot * kLatent + d], acc);
    }
    out[((int64_t)t * H + h) * kLatent + d] = acc * inv;
  }
}

int pick_splits(int T, int H, int max_entries) {
  // Aim for ~1024 waves in flight, each split at least two tiles long.
  const int nw = H / 16;
  const int max_split = (max_entries + 2 * kTile - 1) / (2 * kTile);
  int s = (1024 + T * nw - 1) / (T * nw);
  if (s > max_split) s = max_split;
  return s < 1 ? 1 : s;
}

}  // namespace

size_t attention_ws_bytes(int64_t T, int64_t max_entries, int H) {
  const int s = pick_splits((int)T, H, (int)max_entries);
  if (s <= 1) return 0;
  return (size_t)T * s * H * (kLatent + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int max_entries = a.max_comp + a.window;
  if (a.comp.fmt == CSA_F32) {
    const size_t lds = (kKvDim + max_entries + 8) * sizeof(float);
    hipLaunchKernelGGL(attn_f32_kernel, dim3(a.H, a.T), dim3(256), lds, s, (const float*)a.q,
                       a.H, a.q_seq, a.q_pos, a.hca, a.phys_idx, a.k_sel, a.ratio, a.comp, a.comp_pt,
                       a.comp_pt_stride, a.raw, a.raw_pt, a.raw_pt_stride, a.window, a.scale,
                       (float*)a.out);
    return hipGetLastError();
  }
  const int nsplit = pick_splits(a.T, a.H, max_entries);
  int split_len = (max_entries + nsplit - 1) / nsplit;
  split_len = ((split_len + kTile - 1) / kTile) * kTile;
  const bool f32o = a.out_fmt == CSA_F32;
  float* part = nsplit > 1 ? (float*)a.ws : nullptr;
  const int nw = a.H >= 64 ? 4 : a.H / 16;  // waves per workgroup (16 heads each)
  dim3 grid(nsplit, a.T, a.H / (16 * nw));
#define CSA_ATTN(NW, FO)                                                                   \
  hipLaunchKernelGGL((attn_mfma_kernel<NW, FO>), grid, dim3(NW * 64), 0, s,               \
                     (const uint16_t*)a.q, a.H, a.q_seq, a.q_pos, a.hca, a.phys_idx, a.k_sel, \
                     a.ratio, a.comp, a.comp_pt, a.comp_pt_stride, a.raw, a.raw_pt,      \
                     a.raw_pt_stride, a.window, a.scale, a.out, part, split_len, nsplit)
  if (nw == 4) { if (f32o) CSA_ATTN(4, true); else CSA_ATTN(4, false); }
  else if (nw == 2) { if (f32o) CSA_ATTN(2, true); else CSA_ATTN(2, false); }
  else { if (f32o) CSA_ATTN(1, true); else CSA_ATTN(1, false); }
#undef CSA_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  if (f32o)
    hipLaunchKernelGGL(attn_combine_kernel<true>, dim3(a.H, a.T), dim3(256), 0, s, part, a.T,
                       a.H, nsplit, a.out);
  else
    hipLaunchKernelGGL(attn_combine_kernel<false>, dim3(a.H, a.T), dim3(256), 0, s, part, a.T,
                       a.H, nsplit, a.out);
  return hipGetLastError();
}

}  // namespace csa
