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
  csa_index_pool kpool;
  void* q_out;
  void* q_out_scale;
};
hipError_t launch_decode_prep(const DecodePrepArgs& a, hipStream_t s);

hipError_t launch_index_prep(const void* v, int v_fmt, int64_t rows, int dim, uint32_t flags,
                             int out_fmt, void* out, void* out_scale, const int32_t* dst_rows,
                             hipStream_t s);

hipError_t launch_indexer(const void* q, int q_fmt, const void* q_scale, uint32_t prep,
                          const float* w, int T, int H_I, int D_I, const int32_t* row_seq,
                          const int32_t* row_len, int max_row_len, const int32_t* page_table,
                          int pt_stride, const csa_index_pool& k, float* logits, int64_t ld,
                          void* q_used, void* q_used_scale, void* ws, hipStream_t s,
                          uint32_t* okeys = nullptr, int32_t* ojs = nullptr,
                          int32_t* ophys = nullptr);

// Candidates per row the final top-512 pass takes in one workgroup (16 keys
// per lane at 1024 threads). Rows with more scan chunks first merge groups of
// chunks into at most kCandGroups lists (each group at most kCandFinalMax
// candidates), so the fused path takes up to kCandGroups * 32 chunks per row.
constexpr int kCandFinalMax = 16384;
constexpr int kCandGroups = 8;
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

hipError_t launch_topk(const float* logits, int64_t ld, int R, const int32_t* row_len,
                       const int32_t* row_seq, const int32_t* page_table, int pt_stride,
                       int c4_page_size, int max_row_len, int32_t* phys_idx,
                       int32_t* logical_idx, void* ws, hipStream_t s);

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
size_t topk_ws_bytes(int64_t R, int64_t max_len);
int64_t topk_max_len();
size_t indexer_ws_bytes(int64_t T, int H_I);
size_t indexer_topk_ws_bytes(int64_t T, int64_t max_row_len, int H_I);

}  // namespace csa
