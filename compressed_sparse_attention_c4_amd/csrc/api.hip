// api.hip -- the extern "C" entry points declared in include/csa.h: host-side
// argument checks (before any launch), then the kernel launchers.
#include <hip/hip_runtime.h>

#include <limits.h>

#include <algorithm>
#include <mutex>

#include "../../include/csa.h"
#include "csa_internal.hpp"

using namespace csa;

namespace {

inline csa_status hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

inline bool kv_pool_ok(const csa_kv_pool& p) {
  if (!p.latent || !p.rope || p.page_size <= 0 || p.num_pages < 0) return false;
  if (p.fmt == CSA_FP8_E4M3) return p.latent_scale != nullptr;
  return p.fmt == CSA_F32;
}

// Argument checks shared by indexer_score and indexer_topk512 (everything but
// the output); CSA_OK when the call may proceed.
csa_status indexer_args(csa_fmt q_fmt, const void* q_scale, uint32_t prep, int32_t T, int32_t H_I,
                        int32_t D_I, int32_t max_row_len, int32_t pt_stride,
                        const csa_index_pool& k, const void* q_used, const void* q_used_scale,
                        const void* ws, size_t ws_bytes) {
  if (T < 0 || H_I <= 0 || max_row_len < 0 || pt_stride <= 0) return CSA_ERR_INVALID;
  if (k.page_size <= 0 || k.dim != D_I) return CSA_ERR_INVALID;
  if ((q_used == nullptr) != (q_used_scale == nullptr)) return CSA_ERR_INVALID;
  if (prep & ~(CSA_PREP_HADAMARD | CSA_PREP_QUANT | CSA_ROWS_PER_SEQ(0xFF))) return CSA_ERR_INVALID;
  const uint32_t prep_ops = prep & (CSA_PREP_HADAMARD | CSA_PREP_QUANT);
  if (k.fmt == CSA_F32) {
    if (q_fmt != CSA_F32 || prep_ops != 0) return CSA_ERR_INVALID;
    if (D_I != 64 && D_I != 128) return CSA_ERR_UNSUPPORTED;
    if ((size_t)H_I * D_I > 8192) return CSA_ERR_UNSUPPORTED;
    if (q_used) return CSA_ERR_INVALID;
  } else if (k.fmt == CSA_FP8_E4M3 || k.fmt == CSA_MXFP4) {
    if (H_I != 64 || D_I != 128) return CSA_ERR_UNSUPPORTED;
    if (k.page_size % 16 != 0) return CSA_ERR_UNSUPPORTED;
    if (!k.scale) return CSA_ERR_INVALID;
    if (q_fmt == CSA_BF16 || q_fmt == CSA_F32) {
      if (!(prep_ops & CSA_PREP_QUANT)) return CSA_ERR_INVALID;
      if (!q_used && ws_bytes < indexer_ws_bytes(T, H_I)) return CSA_ERR_WORKSPACE;
      if (!q_used && !ws) return CSA_ERR_WORKSPACE;
    } else if (q_fmt == k.fmt) {
      if (prep_ops != 0 || !q_scale) return CSA_ERR_INVALID;
    } else {
      return CSA_ERR_INVALID;
    }
  } else {
    return CSA_ERR_INVALID;
  }
  return CSA_OK;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// A rotary embedding description used with CSA_PREP_ROPE on rows of `dim`.
inline bool rope_ok(const csa_rope& r, int dim, bool need_groups) {
  if (!r.pos || !r.cos_sin) return false;
  if (r.dim < 2 || r.dim > dim || (r.dim & 1)) return false;
  return !need_groups || r.rows_per_pos >= 1;
}

// indexer_topk512's workspace: the query-preparation area, then either the
// scan's top-512 candidates (fused path) or the logits and the top-512
// workspace (two-call path); sized for whichever is larger.
// Layout: [the fused finish's counters, fixed size][query preparation][...].
struct IdxTopkWs {
  size_t ctr, prep, cand, merged, logits, topk, rsel, total;
  int64_t ld;
};
IdxTopkWs idx_topk_ws(int64_t T, int64_t max_row_len, int H_I) {
  IdxTopkWs w{};
  w.ctr = align256(kCandCounterBytes);
  w.prep = w.ctr + align256(indexer_ws_bytes(T, H_I));
  const int64_t chunks = indexer_scan_chunks(T, max_row_len);
  w.cand = align256((size_t)T * chunks * CSA_TOPK * sizeof(uint32_t));
  w.merged = align256((size_t)T * kCandGroups * CSA_TOPK * sizeof(uint32_t));
  w.ld = std::max<int64_t>(64, (max_row_len + 63) / 64 * 64);
  w.logits = align256((size_t)T * w.ld * sizeof(float));
  w.topk = align256(topk_ws_bytes(T, w.ld, CSA_TOPK));
  // the row-block selection's per-range candidates (several page ranges)
  w.rsel = align256((size_t)T * indexer_rows_sel_cands(T, max_row_len) * sizeof(uint32_t));
  w.total = w.prep + std::max({3 * (w.cand + w.merged), w.logits + w.topk, 3 * w.rsel});
  return w;
}

}  // namespace

namespace csa {
size_t indexer_topk_ws_bytes(int64_t T, int64_t max_row_len, int H_I) {
  return idx_topk_ws(T, max_row_len, H_I).total;
}
}  // namespace csa

extern "C" {

const char* csa_version(void) { return "0.1.0"; }

void csa_set_debug(int32_t on) { set_debug(on); }
int32_t csa_debug_enabled(void) { return debug_on() ? 1 : 0; }

const char* csa_status_string(csa_status s) {
  switch (s) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported format or shape";
    case CSA_ERR_WORKSPACE: return "workspace too small";
    case CSA_ERR_HIP: return "HIP runtime error";
    case CSA_ERR_BOUNDS: return "device data out of range (debug mode)";
  }
  return "unknown status";
}

size_t csa_workspace_size(int32_t op, int64_t rows, int64_t max_len, int32_t heads) {
  if (rows < 0 || max_len < 0 || heads <= 0) return 0;
  switch (op) {
    case CSA_OP_INDEXER: return indexer_ws_bytes(rows, heads);
    case CSA_OP_TOPK: return topk_ws_bytes(rows, max_len, CSA_TOPK);  // max_len = ld
    case CSA_OP_TOPK_K:  // max_len = ld, heads = k
      return heads <= CSA_TOPK_MAX ? topk_ws_bytes(rows, max_len, heads) : 0;
    case CSA_OP_CSA_ATTN:
    case CSA_OP_HCA_ATTN: return attention_ws_bytes(rows, max_len, heads);
    case CSA_OP_CSA_ATTN_F32:
    case CSA_OP_HCA_ATTN_F32: return attention_f32_ws_bytes(rows, max_len, heads);
    case CSA_OP_INDEXER_TOPK: return indexer_topk_ws_bytes(rows, max_len, heads);
    default: return 0;
  }
}

csa_status c4_compress(const void* x, csa_fmt x_fmt, const int32_t* cu_rows,
                       const int32_t* start_pos, int32_t B, int32_t max_rows, int32_t ratio,
                       const float* gate_w, const float* gate_b, const int32_t* page_table,
                       int32_t pt_stride, csa_kv_pool out, hipStream_t stream) {
  if (B < 0 || max_rows < 0 || ratio < 1 || ratio > 1024 || pt_stride <= 0) return CSA_ERR_INVALID;
  if (x_fmt != CSA_BF16 && x_fmt != CSA_F32) return CSA_ERR_INVALID;
  if (!kv_pool_ok(out)) return CSA_ERR_INVALID;
  if (B == 0 || max_rows < ratio) return CSA_OK;
  if (!x || !cu_rows || !start_pos || !gate_w || !gate_b || !page_table) return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d("c4_compress", stream);
    d.rows(kCheckCompress, B, nullptr, start_pos, 0, ratio, 0, cu_rows, page_table, pt_stride,
           out.page_size, out.num_pages);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_compress(x, x_fmt, cu_rows, start_pos, B, max_rows, ratio, gate_w,
                                    gate_b, page_table, pt_stride, out, stream));
}

csa_status csa_index_prep(const void* v, csa_fmt v_fmt, int64_t rows, int32_t dim,
                          uint32_t flags, csa_fmt out_fmt, void* out, void* out_scale,
                          const int32_t* dst_rows, csa_rope rope, hipStream_t stream) {
  if (rows < 0 || (dim != 64 && dim != 128)) return CSA_ERR_INVALID;
  if (v_fmt != CSA_BF16 && v_fmt != CSA_F32) return CSA_ERR_INVALID;
  if (flags & ~(CSA_PREP_HADAMARD | CSA_PREP_QUANT | CSA_PREP_ROPE)) return CSA_ERR_INVALID;
  if ((flags & CSA_PREP_ROPE) && !rope_ok(rope, dim, true)) return CSA_ERR_INVALID;
  if (out_fmt != CSA_F32 && out_fmt != CSA_FP8_E4M3 && out_fmt != CSA_MXFP4) return CSA_ERR_INVALID;
  if (rows == 0) return CSA_OK;
  if (!v || !out || (out_fmt != CSA_F32 && !out_scale)) return CSA_ERR_INVALID;
  return hip_status(launch_index_prep(v, v_fmt, rows, dim, flags, out_fmt, out, out_scale,
                                      dst_rows, rope, stream));
}

csa_status csa_decode_prep(const void* x, csa_fmt x_fmt, const int32_t* pos, int32_t B,
                           int32_t ratio, const float* gate_w, const float* gate_b,
                           const int32_t* page_table, int32_t pt_stride, csa_kv_pool c4,
                           const int32_t* raw_page_table, int32_t raw_pt_stride,
                           csa_kv_pool raw, const void* k_rows, const void* q_rows,
                           csa_fmt kq_fmt, int32_t H_I, uint32_t flags, csa_rope rope,
                           csa_index_pool kpool, void* q_out, void* q_out_scale,
                           hipStream_t stream) {
  if (B < 0 || ratio < 1 || ratio > 128 || pt_stride <= 0 || raw_pt_stride <= 0 || H_I < 0)
    return CSA_ERR_INVALID;
  if (x_fmt != CSA_BF16 && x_fmt != CSA_F32) return CSA_ERR_INVALID;
  if (!kv_pool_ok(c4) || !kv_pool_ok(raw) || c4.fmt != raw.fmt) return CSA_ERR_INVALID;
  if (flags & ~(uint32_t)(CSA_PREP_HADAMARD | CSA_PREP_ROPE)) return CSA_ERR_INVALID;
  const bool kq = k_rows || q_rows;
  if (kq && (flags & CSA_PREP_ROPE)) {
    rope.pos = pos;  // decode rotates at each sequence's token position
    if (!rope_ok(rope, kpool.dim, false)) return CSA_ERR_INVALID;
  }
  if (kq) {
    if (kq_fmt != CSA_BF16 && kq_fmt != CSA_F32) return CSA_ERR_INVALID;
    if (kpool.dim != 64 && kpool.dim != 128) return CSA_ERR_INVALID;
    if (kpool.fmt != CSA_F32 && kpool.fmt != CSA_FP8_E4M3 && kpool.fmt != CSA_MXFP4)
      return CSA_ERR_INVALID;
    if (kpool.fmt != CSA_F32 && !kpool.scale && k_rows) return CSA_ERR_INVALID;
    if (k_rows && (!kpool.data || kpool.page_size != c4.page_size)) return CSA_ERR_INVALID;
    if (q_rows && (!q_out || (kpool.fmt != CSA_F32 && !q_out_scale) || H_I == 0))
      return CSA_ERR_INVALID;
  }
  if (B == 0) return CSA_OK;
  if (!x || !pos || !gate_w || !gate_b || !page_table || !raw_page_table) return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d("csa_decode_prep", stream);
    const int64_t c4_pages = k_rows ? std::min(c4.num_pages, kpool.num_pages) : c4.num_pages;
    d.rows(kCheckDecode, B, nullptr, pos, 0, ratio, 0, nullptr, page_table, pt_stride,
           c4.page_size, c4_pages);
    d.rows(kCheckDecode, B, nullptr, pos, 0, 1, 0, nullptr, raw_page_table, raw_pt_stride,
           raw.page_size, raw.num_pages);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  DecodePrepArgs a{};
  a.x = x; a.x_fmt = x_fmt; a.pos = pos; a.B = B; a.ratio = ratio; a.gate_w = gate_w;
  a.gate_b = gate_b; a.page_table = page_table; a.pt_stride = pt_stride; a.c4 = c4;
  a.raw_page_table = raw_page_table; a.raw_pt_stride = raw_pt_stride; a.raw = raw;
  a.k_rows = k_rows; a.q_rows = q_rows; a.kq_fmt = kq_fmt; a.H_I = H_I; a.flags = flags;
  a.rope = rope;
  a.kpool = kpool; a.q_out = q_out; a.q_out_scale = q_out_scale;
  if (!kq) a.kpool.dim = 128;  // sizes the (unused) row layout only
  return hip_status(launch_decode_prep(a, stream));
}

csa_status indexer_score(const void* q, csa_fmt q_fmt, const void* q_scale, uint32_t prep,
                         const float* w, int32_t T, int32_t H_I, int32_t D_I,
                         const int32_t* row_seq, const int32_t* row_len, int32_t max_row_len,
                         const int32_t* page_table, int32_t pt_stride, csa_index_pool k,
                         float* logits, int64_t ld, void* q_used, void* q_used_scale, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (ld < max_row_len) return CSA_ERR_INVALID;
  const csa_status st = indexer_args(q_fmt, q_scale, prep, T, H_I, D_I, max_row_len, pt_stride, k,
                                     q_used, q_used_scale, ws, ws_bytes);
  if (st != CSA_OK) return st;
  if (T == 0 || max_row_len == 0) return CSA_OK;
  if (!q || !w || !row_seq || !row_len || !page_table || !k.data || !logits) return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d("indexer_score", stream);
    d.rows(kCheckRowLen, T, row_seq, row_len, max_row_len, 1, 0, nullptr, page_table, pt_stride,
           k.page_size, k.num_pages);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_indexer(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len,
                                   max_row_len, page_table, pt_stride, k, logits, ld, q_used,
                                   q_used_scale, ws, stream));
}

csa_status topk_page_select(const float* logits, int64_t ld, int32_t R, const int32_t* row_len,
                            const int32_t* row_seq, const int32_t* page_table, int32_t pt_stride,
                            int32_t page_size, int32_t k, int32_t* phys_idx,
                            int32_t* logical_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (R < 0 || ld < 0 || pt_stride <= 0 || page_size <= 0) return CSA_ERR_INVALID;
  if (k < 1 || k > CSA_TOPK_MAX) return CSA_ERR_INVALID;
  if (ld > topk_max_len(k)) return CSA_ERR_UNSUPPORTED;
  if (R == 0) return CSA_OK;
  if (!logits || !row_len || !row_seq || !page_table || !phys_idx) return CSA_ERR_INVALID;
  const size_t need = topk_ws_bytes(R, ld, k);
  if (need > ws_bytes || (need > 0 && !ws)) return CSA_ERR_WORKSPACE;
  if (debug_on()) {  // (no pool here: page ids are checked against their sign only)
    DebugCheck d("topk_page_select", stream);
    d.rows(kCheckRowLen, R, row_seq, row_len, ld, 1, 0, nullptr, page_table, pt_stride, page_size,
           INT32_MAX);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_topk(logits, ld, R, row_len, row_seq, page_table, pt_stride, page_size,
                                k, phys_idx, logical_idx, ws, stream));
}

csa_status topk512_page_select(const float* logits, int64_t ld, int32_t R,
                               const int32_t* row_len, const int32_t* row_seq,
                               const int32_t* page_table, int32_t pt_stride,
                               int32_t c4_page_size, int32_t* phys_idx, int32_t* logical_idx,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  return topk_page_select(logits, ld, R, row_len, row_seq, page_table, pt_stride, c4_page_size,
                          CSA_TOPK, phys_idx, logical_idx, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// indexer_topk512 with its workspace given (a caller's buffer, or the
// library's own scratch array for indexer_topk512_noalloc).
csa_status indexer_topk512_ws(const void* q, csa_fmt q_fmt, const void* q_scale, uint32_t prep,
                              const float* w, int32_t T, int32_t H_I, int32_t D_I,
                              const int32_t* row_seq, const int32_t* row_len, int32_t max_row_len,
                              const int32_t* page_table, int32_t pt_stride, csa_index_pool k,
                              int32_t* phys_idx, int32_t* logical_idx, void* q_used,
                              void* q_used_scale, void* ws, size_t ws_bytes, hipEvent_t scan_done,
                              hipStream_t stream) {
  const csa_status st = indexer_args(q_fmt, q_scale, prep, T, H_I, D_I, max_row_len, pt_stride, k,
                                     q_used, q_used_scale, ws, ws_bytes);
  if (st != CSA_OK) return st;
  if (max_row_len > topk_max_len(CSA_TOPK)) return CSA_ERR_UNSUPPORTED;
  if (T == 0) return CSA_OK;
  const IdxTopkWs L = idx_topk_ws(T, max_row_len, H_I);
  if (!ws || ws_bytes < L.total) return CSA_ERR_WORKSPACE;
  if (!q || !w || !row_seq || !row_len || !page_table || !k.data || !phys_idx) return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d("indexer_topk512", stream);
    d.rows(kCheckRowLen, T, row_seq, row_len, max_row_len, 1, 0, nullptr, page_table, pt_stride,
           k.page_size, k.num_pages);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  uint8_t* base = (uint8_t*)ws;
  uint8_t* prep_ws = base + L.ctr;  // the prepared query, when prepared in the call
  const int chunks = indexer_cand_chunks(T, H_I, D_I, k, max_row_len, prep);
  const int ranges = indexer_rows_sel_ranges(T, H_I, D_I, k, max_row_len, prep);
  hipError_t e;
  if (ranges > 0) {
    // many rows per sequence: the row-block kernel keeps each row's top-512
    // as it scores; with several page ranges per row a final pass merges the
    // ranges' candidates
    CandOut co{};
    co.rows_sel = 1;
    co.phys_idx = phys_idx;
    co.logical_idx = logical_idx;
    co.keys = (uint32_t*)(base + L.prep);
    co.js = (int32_t*)(base + L.prep + L.rsel);
    co.phys = (int32_t*)(base + L.prep + 2 * L.rsel);
    e = launch_indexer(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len, max_row_len,
                       page_table, pt_stride, k, nullptr, 0, q_used, q_used_scale, prep_ws, stream,
                       &co);
    if (e == hipSuccess && scan_done) e = hipEventRecord(scan_done, stream);
    if (e == hipSuccess && ranges > 1)
      e = launch_topk_cand_final(co.keys, co.js, co.phys, ranges * CSA_TOPK, T, row_len, row_seq,
                                 page_table, pt_stride, k.page_size, phys_idx, logical_idx, stream);
  } else if (chunks > 0) {
    CandOut co{};
    co.keys = (uint32_t*)(base + L.prep);
    co.js = (int32_t*)(base + L.prep + L.cand);
    co.phys = (int32_t*)(base + L.prep + 2 * L.cand);
    uint32_t* mk = (uint32_t*)(base + L.prep + 3 * L.cand);
    int32_t* mj = (int32_t*)(base + L.prep + 3 * L.cand + L.merged);
    int32_t* mp = (int32_t*)(base + L.prep + 3 * L.cand + 2 * L.merged);
    // rows of 9..64 chunks finish their selection inside the scan (groups of
    // at most 8 chunks, at most 8 groups), which saves the merge launch; with
    // at most 8 chunks a row goes straight to the final pass
    if (chunks > kCandGroups && chunks <= kCandFusedChunks && T < kCandFusedRows) {
      co.cnt = (uint32_t*)base;
      co.gsize = (chunks + kCandGroups - 1) / kCandGroups;
      co.ngroups = (chunks + co.gsize - 1) / co.gsize;
      co.mkeys = mk;
      co.mjs = mj;
      co.mphys = mp;
      co.phys_idx = phys_idx;
      co.logical_idx = logical_idx;
    }
    e = launch_indexer(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len, max_row_len,
                       page_table, pt_stride, k, nullptr, 0, q_used, q_used_scale, prep_ws, stream,
                       &co);
    if (e == hipSuccess && scan_done) e = hipEventRecord(scan_done, stream);
    if (co.ngroups > 0) return hip_status(e);
    uint32_t* ck = co.keys;
    int32_t* cj = co.js;
    int32_t* cp = co.phys;
    int ncand = chunks * CSA_TOPK;
    if (e == hipSuccess && ncand > kCandFinalMax) {
      // groups of g consecutive chunks -> at most kCandGroups lists
      const int g = (chunks + kCandGroups - 1) / kCandGroups;
      const int groups = (chunks + g - 1) / g;
      e = launch_topk_cand_merge(ck, cj, cp, ncand, g * CSA_TOPK, T, row_len, mk, mj, mp, stream);
      ck = mk;
      cj = mj;
      cp = mp;
      ncand = groups * CSA_TOPK;
    }
    if (e == hipSuccess)
      e = launch_topk_cand_final(ck, cj, cp, ncand, T, row_len, row_seq, page_table, pt_stride,
                                 k.page_size, phys_idx, logical_idx, stream);
  } else {
    float* logits = (float*)(base + L.prep);
    e = launch_indexer(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len, max_row_len,
                       page_table, pt_stride, k, logits, L.ld, q_used, q_used_scale, prep_ws, stream);
    if (e == hipSuccess && scan_done) e = hipEventRecord(scan_done, stream);
    if (e == hipSuccess)
      e = launch_topk(logits, L.ld, T, row_len, row_seq, page_table, pt_stride, k.page_size,
                      CSA_TOPK, phys_idx, logical_idx, base + L.prep + L.logits, stream);
  }
  return hip_status(e);
}

// The library's own workspace for callers that cannot allocate: one array per
// GPU in device memory, held until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and is what the kernels receive.
constexpr size_t kScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array (nullptr on failure).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

csa_status indexer_topk512(const void* q, csa_fmt q_fmt, const void* q_scale, uint32_t prep,
                           const float* w, int32_t T, int32_t H_I, int32_t D_I,
                           const int32_t* row_seq, const int32_t* row_len, int32_t max_row_len,
                           const int32_t* page_table, int32_t pt_stride, csa_index_pool k,
                           int32_t* phys_idx, int32_t* logical_idx, void* q_used,
                           void* q_used_scale, void* ws, size_t ws_bytes, hipEvent_t scan_done,
                           hipStream_t stream) {
  return indexer_topk512_ws(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len, max_row_len,
                            page_table, pt_stride, k, phys_idx, logical_idx, q_used, q_used_scale,
                            ws, ws_bytes, scan_done, stream);
}

csa_status indexer_topk512_noalloc(const void* q, csa_fmt q_fmt, const void* q_scale,
                                   uint32_t prep, const float* w, int32_t T, int32_t H_I,
                                   int32_t D_I, const int32_t* row_seq, const int32_t* row_len,
                                   int32_t max_row_len, const int32_t* page_table,
                                   int32_t pt_stride, csa_index_pool k, int32_t* phys_idx,
                                   int32_t* logical_idx, void* q_used, void* q_used_scale,
                                   hipStream_t stream) {
  if (T < 0 || max_row_len < 0 || H_I <= 0) return CSA_ERR_INVALID;
  if (max_row_len > topk_max_len(CSA_TOPK)) return CSA_ERR_UNSUPPORTED;
  if (indexer_topk_ws_bytes(T, max_row_len, H_I) > kScratchBytes) return CSA_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return CSA_ERR_HIP;
  return indexer_topk512_ws(q, q_fmt, q_scale, prep, w, T, H_I, D_I, row_seq, row_len, max_row_len,
                            page_table, pt_stride, k, phys_idx, logical_idx, q_used, q_used_scale,
                            ws, kScratchBytes, nullptr, stream);
}

csa_status hisparse_swap_in(const int32_t* logical_idx, int32_t R, int32_t k,
                            const int32_t* row_seq, csa_kv_pool far,
                            const int32_t* far_page_table, int32_t far_pt_stride,
                            csa_kv_pool near, int32_t hot_slots, int32_t* slot_of,
                            int64_t max_entries, int32_t* owner, int32_t* last_use, int32_t step,
                            int32_t* near_idx, hipStream_t stream) {
  if (R < 0 || k < 1 || k > hisparse_max_sel() || far_pt_stride <= 0) return CSA_ERR_INVALID;
  if (hot_slots < k || hot_slots > hisparse_max_hot()) return CSA_ERR_INVALID;
  if (max_entries < 1 || step < 0) return CSA_ERR_INVALID;
  if (!kv_pool_ok(far) || !kv_pool_ok(near) || far.fmt != near.fmt) return CSA_ERR_INVALID;
  if (R == 0) return CSA_OK;
  if (!logical_idx || !row_seq || !far_page_table || !slot_of || !owner || !last_use || !near_idx)
    return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d("hisparse_swap_in", stream);
    d.idx((int64_t)R * k, k, logical_idx, max_entries, kBadEntry);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_hisparse_swap(logical_idx, R, k, row_seq, far, far_page_table,
                                         far_pt_stride, near, hot_slots, slot_of, max_entries,
                                         owner, last_use, step, near_idx, stream));
}

static csa_status attn_common(AttnArgs& a, hipStream_t stream) {
  if (a.T < 0 || a.H <= 0 || a.window < 0 || a.window > 4096) return CSA_ERR_INVALID;
  if (!a.hca && a.k_sel + a.window < 1) return CSA_ERR_INVALID;
  if (a.hca && a.window < 1) return CSA_ERR_INVALID;
  if (!kv_pool_ok(a.comp) || !kv_pool_ok(a.raw) || a.comp.fmt != a.raw.fmt) return CSA_ERR_INVALID;
  if (a.raw_pt_stride <= 0) return CSA_ERR_INVALID;
  if (a.comp.fmt == CSA_F32) {
    if (a.q_fmt != CSA_F32 || a.out_fmt != CSA_F32) return CSA_ERR_INVALID;
    if ((int64_t)a.max_comp + a.window > 32768) return CSA_ERR_UNSUPPORTED;
    const size_t need = attention_f32_ws_bytes(a.T, a.max_comp + a.window, a.H);
    if (need > a.ws_bytes || (need > 0 && !a.ws)) return CSA_ERR_WORKSPACE;
  } else {
    if (a.q_fmt != CSA_BF16) return CSA_ERR_INVALID;
    if (a.out_fmt != CSA_BF16 && a.out_fmt != CSA_F32) return CSA_ERR_INVALID;
    if (a.H % 16 != 0 || a.H == 48 || (a.H > 64 && a.H % 64 != 0) || a.H > 1024) return CSA_ERR_UNSUPPORTED;
    const size_t need = attention_ws_bytes(a.T, a.max_comp + a.window, a.H);
    if (need > a.ws_bytes || (need > 0 && !a.ws)) return CSA_ERR_WORKSPACE;
  }
  if (a.T == 0) return CSA_OK;
  if (!a.q || !a.q_seq || !a.q_pos || !a.raw_pt || !a.out) return CSA_ERR_INVALID;
  if (debug_on()) {
    DebugCheck d(a.hca ? "hca_dense_attn" : "csa_sparse_attn", stream);
    if (a.hca)
      d.rows(kCheckHca, a.T, a.q_seq, a.q_pos, 0, a.ratio, 0, nullptr, a.comp_pt,
             a.comp_pt_stride, a.comp.page_size, a.comp.num_pages);
    else if (a.k_sel > 0)
      d.idx((int64_t)a.T * a.k_sel, a.k_sel, a.phys_idx, a.comp.num_pages * a.comp.page_size,
            kBadSlot);
    d.rows(kCheckWindow, a.T, a.q_seq, a.q_pos, 0, 1, a.window, nullptr, a.raw_pt,
           a.raw_pt_stride, a.raw.page_size, a.raw.num_pages);
    const csa_status st = d.result();
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_attention(a, stream));
}

csa_status csa_sparse_attn(const void* q, csa_fmt q_fmt, int32_t T, int32_t H,
                           const int32_t* q_seq, const int32_t* q_pos, const int32_t* phys_idx,
                           int32_t k_sel, csa_kv_pool c4, csa_kv_pool raw,
                           const int32_t* raw_page_table, int32_t raw_pt_stride, int32_t window,
                           float softmax_scale, void* out, csa_fmt out_fmt, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (k_sel < 0 || k_sel > CSA_TOPK_MAX) return CSA_ERR_INVALID;
  if (k_sel > 0 && !phys_idx && T > 0) return CSA_ERR_INVALID;
  AttnArgs a{};
  a.q = q; a.q_fmt = q_fmt; a.T = T; a.H = H; a.q_seq = q_seq; a.q_pos = q_pos;
  a.hca = false; a.phys_idx = phys_idx; a.k_sel = k_sel; a.ratio = 1; a.comp = c4; a.comp_pt = nullptr;
  a.comp_pt_stride = 1; a.max_comp = k_sel; a.raw = raw; a.raw_pt = raw_page_table;
  a.raw_pt_stride = raw_pt_stride; a.window = window; a.scale = softmax_scale; a.out = out;
  a.out_fmt = out_fmt; a.ws = ws; a.ws_bytes = ws_bytes;
  return attn_common(a, stream);
}

csa_status hca_dense_attn(const void* q, csa_fmt q_fmt, int32_t T, int32_t H,
                          const int32_t* q_seq, const int32_t* q_pos, int32_t max_len,
                          int32_t ratio, csa_kv_pool hca, const int32_t* hca_page_table,
                          int32_t hca_pt_stride, csa_kv_pool raw, const int32_t* raw_page_table,
                          int32_t raw_pt_stride, int32_t window, float softmax_scale, void* out,
                          csa_fmt out_fmt, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ratio < 1 || max_len < 0 || hca_pt_stride <= 0) return CSA_ERR_INVALID;
  if (T > 0 && !hca_page_table) return CSA_ERR_INVALID;
  AttnArgs a{};
  a.q = q; a.q_fmt = q_fmt; a.T = T; a.H = H; a.q_seq = q_seq; a.q_pos = q_pos;
  a.hca = true; a.phys_idx = nullptr; a.k_sel = 0; a.ratio = ratio; a.comp = hca; a.comp_pt = hca_page_table;
  a.comp_pt_stride = hca_pt_stride; a.max_comp = max_len / ratio; a.raw = raw;
  a.raw_pt = raw_page_table; a.raw_pt_stride = raw_pt_stride; a.window = window;
  a.scale = softmax_scale; a.out = out; a.out_fmt = out_fmt; a.ws = ws; a.ws_bytes = ws_bytes;
  return attn_common(a, stream);
}

}  // extern "C"
