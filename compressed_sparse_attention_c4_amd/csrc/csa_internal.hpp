// csa_internal.hpp -- launch functions behind the C ABI (host side, internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Each launcher enqueues on `s` and returns hipGetLastError().
hipError_t launch_compress(const void* x, int x_fmt, const int32_t* cu_rows,
                           const int32_t* start_pos, int B, int max_rows, int ratio,
                           const float* gate_w, const float* gate_b,
                           const int32_t* page_table, int pt_stride, const csa_kv_pool& out,
                           hipStream_t s);

struct DecodePrepArgs {
  const void* x;  // [B][ratio][576]
  int x_fmt;
  const int32_t* pos;
  int B, ratio;
  const float* gate_w;
  const float* gate_b;
  const int32_t* page_table;  // c4 pool and index pool (same entries, same page size)
  int pt_stride;
  csa_kv_pool c4;
  const int32_t* raw_page_table;
  int raw_pt_stride;
  csa_kv_pool raw;
  const void* k_rows;  // [B][dim] or NULL
  const void* q_rows;  // [B][H_I][dim] or NULL
  int kq_fmt;
  int H_I;
  uint32_t flags;
  csa_rope rope;
  csa_index_pool kpool;
  void* q_out;
  void* q_out_scale;
};
hipError_t launch_decode_prep(const DecodePrepArgs& a, hipStream_t s);

hipError_t launch_index_prep(const void* v, int v_fmt, int64_t rows, int dim, uint32_t flags,
                             int out_fmt, void* out, void* out_scale, const int32_t* dst_rows,
                             const csa_rope& rope, hipStream_t s);

// Where the fused decode scan puts its top-512 candidates (indexer_topk512).
// Each scan workgroup writes its chunk's candidates (keys, js, phys: [T][chunks]
// [512]). With ngroups > 0 the selection also finishes inside the scan: the
// last workgroup of each group of gsize chunks (found with a counter in cnt)
// merges the group's candidates, into mkeys / mjs / mphys [T][ngroups][512]
// when ngroups > 1, and the last group of a row selects the row's top-512 into
// phys_idx / logical_idx. cnt [T][kCandGroups + 1] must hold zeros; every
// counter is returned to zero by the workgroup that completes it.
// With rows_sel the row-block kernel selects instead (8 rows per workgroup,
// the ranges given by indexer_rows_sel_ranges): one range writes phys_idx /
// logical_idx, several write keys / js / phys [T][ranges][512] for
// launch_topk_cand_final.
struct CandOut {
  uint32_t* keys;
  int32_t* js;
  int32_t* phys;
  uint32_t* cnt;
  int gsize, ngroups;
  uint32_t* mkeys;
  int32_t* mjs;
  int32_t* mphys;
  int32_t* phys_idx;
  int32_t* logical_idx;
  int rows_sel;
  int wide_rows, wide_chunks;  // set by launch_indexer for a long ragged batch's scan
};

hipError_t launch_indexer(const void* q, int q_fmt, const void* q_scale, uint32_t prep,
                          const float* w, int T, int H_I, int D_I, const int32_t* row_seq,
                          const int32_t* row_len, int max_row_len, const int32_t* page_table,
                          int pt_stride, const csa_index_pool& k, float* logits, int64_t ld,
                          void* q_used, void* q_used_scale, void* ws, hipStream_t s,
                          const CandOut* cand = nullptr);

// Candidates per row the final top-512 pass takes in one workgroup (16 keys
// per lane at 1024 threads). Rows with more scan chunks first merge groups of
// chunks into at most kCandGroups lists (each group at most kCandFinalMax
// candidates), so the fused path takes up to kCandGroups * 32 chunks per row.
constexpr int kCandFinalMax = 16384;
constexpr int kCandGroups = 8;
// The fused finish inside the scan takes groups of at most 4096 candidates
// (8 chunks), so rows of at most kCandGroups * 8 chunks; rows of fewer than
// kCandFusedRows rows. Its counters sit at the start of the workspace, in a
// region of fixed size, so that calls of any shape find them where the last
// call left them (zero).
constexpr int kCandFusedChunks = kCandGroups * 8;
constexpr int kCandFusedRows = 256;
constexpr size_t kCandCounterBytes = (size_t)kCandFusedRows * (kCandGroups + 1) * sizeof(uint32_t);
// Fused indexer + top-512: the scan workgroups select their chunk's top-512
// candidates (launch_indexer with okeys / ojs / ophys: key, entry index and
// physical slot), then one final pass per row, which takes the slots from the
// candidates instead of looking them up.
// Returns the scan chunks per row, or 0 when the shapes need the two calls.
// `prep` carries the rows-per-sequence hint, which may route the rows to the
// row-block kernel (two calls).
int indexer_cand_chunks(int64_t T, int H_I, int D_I, const csa_index_pool& k,
                        int64_t max_row_len, uint32_t prep);
// Chunks per row of the decode scan kernel for these sizes.
int64_t indexer_scan_chunks(int64_t T, int64_t max_row_len);
// Page ranges of the row-block kernel's fused selection for this call, or 0
// when the call does not take it (it takes 8 rows per workgroup).
int indexer_rows_sel_ranges(int64_t T, int H_I, int D_I, const csa_index_pool& k,
                            int64_t max_row_len, uint32_t prep);
// Largest ranges * 512 candidates per row that calls of these sizes can need.
int64_t indexer_rows_sel_cands(int64_t T, int64_t max_row_len);
// A row's candidates in groups of `group` (a multiple of 512) reduced to one
// top-512 list per group (okeys / ojs / ophys: R x groups x 512).
hipError_t launch_topk_cand_merge(const uint32_t* ckeys, const int32_t* cjs, const int32_t* cphys,
                                  int ncand, int group, int R, const int32_t* row_len,
                                  uint32_t* okeys, int32_t* ojs, int32_t* ophys, hipStream_t s);
hipError_t launch_topk_cand_final(const uint32_t* ckeys, const int32_t* cjs, const int32_t* cphys,
                                  int ncand, int R,
                                  const int32_t* row_len, const int32_t* row_seq,
                                  const int32_t* page_table, int pt_stride, int c4_page_size,
                                  int32_t* phys_idx, int32_t* logical_idx, hipStream_t s);

// Top-k (1 <= k <= 2048) of each row's logits, translated through the page
// table; rows of phys_idx / logical_idx hold k entries.
hipError_t launch_topk(const float* logits, int64_t ld, int R, const int32_t* row_len,
                       const int32_t* row_seq, const int32_t* page_table, int pt_stride,
                       int c4_page_size, int k, int32_t* phys_idx, int32_t* logical_idx, void* ws,
                       hipStream_t s);

// HiSparse staging of one step's selected entries into the per-sequence hot
// slots of the near pool (see hisparse.hip).
hipError_t launch_hisparse_swap(const int32_t* sel, int R, int k, const int32_t* row_seq,
                                const csa_kv_pool& far, const int32_t* far_pt, int far_pt_stride,
                                const csa_kv_pool& near, int hot, int32_t* slot_of,
                                int64_t max_entries, int32_t* owner, int32_t* last_use, int step,
                                int32_t* near_idx, hipStream_t s);
int hisparse_max_hot();
int hisparse_max_sel();

// Debug mode (debug_check.hip): device-side checks of the integers a call
// follows, run before its kernels; result() synchronises the stream and
// returns CSA_ERR_BOUNDS on a violation (printed to stderr).
bool debug_on();
void set_debug(int on);
enum CheckMode { kCheckRowLen = 0, kCheckWindow = 1, kCheckHca = 2, kCheckCompress = 3,
                 kCheckDecode = 4 };
enum CheckCode { kBadRowLen = 1, kBadPosition = 2, kBadSequence = 3, kBadTableWidth = 4,
                 kBadPage = 5, kBadSlot = 6, kBadEntry = 7 };
class DebugCheck {
 public:
  DebugCheck(const char* entry, hipStream_t s);
  // rows r < R: entry range by mode (kCheckRowLen: [0, lens[r]) with
  // lens[r] <= cap; kCheckWindow: the `window` positions up to lens[r];
  // kCheckHca: [0, (lens[r] + 1) / ratio); kCheckCompress: the entries the
  // rows cu_rows[r]..cu_rows[r+1] starting at position lens[r] complete;
  // kCheckDecode: the entry position lens[r] completes), sequence row_seq[r]
  // (or r), pages of that range in pt, each in [0, num_pages)
  void rows(int mode, int R, const int32_t* row_seq, const int32_t* lens, int64_t cap, int ratio,
            int window, const int32_t* cu_rows, const int32_t* pt, int pt_stride, int page_size,
            int64_t num_pages);
  // n values of v (rows of k): each -1 or in [0, limit)
  void idx(int64_t n, int k, const int32_t* v, int64_t limit, int32_t code);
  csa_status result();

 private:
  const char* entry_;
  hipStream_t s_;
  int32_t* rec_ = nullptr;
  hipError_t err_ = hipSuccess;
};

struct AttnArgs {
  const void* q;
  int q_fmt;
  int T, H;
  const int32_t* q_seq;
  const int32_t* q_pos;
  // compressed part: CSA selects through phys_idx; HCA takes every visible entry
  bool hca;
  const int32_t* phys_idx;  // CSA: [T][k_sel]; NULL for HCA
  int k_sel;
  int ratio;                // HCA: visible entries (p+1)/ratio
  csa_kv_pool comp;
  const int32_t* comp_pt;   // HCA page table
  int comp_pt_stride;
  int max_comp;             // upper bound of compressed entries per query
  csa_kv_pool raw;
  const int32_t* raw_pt;
  int raw_pt_stride;
  int window;
  float scale;
  void* out;
  int out_fmt;
  void* ws;
  size_t ws_bytes;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
size_t attention_ws_bytes(int64_t T, int64_t max_entries, int H);
size_t attention_f32_ws_bytes(int64_t T, int64_t max_entries, int H);
size_t topk_ws_bytes(int64_t R, int64_t max_len, int k);
int64_t topk_max_len(int k);
size_t indexer_ws_bytes(int64_t T, int H_I);
size_t indexer_topk_ws_bytes(int64_t T, int64_t max_row_len, int H_I);

}  // namespace csa
