// debug_check.hip -- the library's debug mode: device-side checks of the
// device-resident integers a call is about to follow (page ids, row lengths,
// positions, selected slots), run on the call's stream before its kernels.
//
// The host cannot read those integers without a synchronisation, so normally a
// page id outside its pool is a breach of the caller's contract with undefined
// results. In debug mode (csa_set_debug(1), or CSA_DEBUG=1 in the environment
// when the library is loaded) each checked entry point first launches the
// checks below, which record the first violation in a small device record
// (code, row, index, value), copies the record back, synchronises the stream
// and, on a violation, prints it to stderr and returns CSA_ERR_BOUNDS without
// launching the call's own kernels. Debug mode synchronises, so it is not for
// graph capture or for timing.
//
// Every check reads only the caller's integers inside the extents the call's
// host-side arguments give (rows, strides, k), and a page-table row is read
// only after its sequence index has been checked to be non-negative; a row of
// a page table past the caller's last sequence is outside what the library
// can know and is not checked.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "csa_internal.hpp"

namespace csa {
namespace {

// The record: [0] violation code (0: none), [1] row, [2] index, [3] value.
static __device__ __align__(16) int32_t g_record[4];

__device__ void report(int32_t code, int32_t row, int32_t index, int32_t value) {
  if (atomicCAS(&g_record[0], 0, code) == 0) {
    g_record[1] = row;
    g_record[2] = index;
    g_record[3] = value;
  }
}

__global__ void record_clear_kernel(int32_t* rec) {
  if (threadIdx.x < 4) rec[threadIdx.x] = 0;
}

// One workgroup per row r: the row's entry range [lo, hi) (by `mode`), its
// sequence s (row_seq[r], or r), the pages of that range in s's page-table
// row, each in [0, num_pages).
__global__ void __launch_bounds__(256)
check_rows_kernel(int mode, int R, const int32_t* __restrict__ row_seq,
                  const int32_t* __restrict__ lens, int64_t cap, int ratio, int window,
                  const int32_t* __restrict__ cu_rows, const int32_t* __restrict__ pt,
                  int pt_stride, int page_size, int64_t num_pages) {
  const int r = blockIdx.x;
  if (r >= R) return;
  const int s = row_seq ? row_seq[r] : r;
  int64_t lo = 0, hi = 0;
  if (mode == kCheckRowLen) {
    const int32_t n = lens[r];
    if (n < 0 || n > cap) {
      if (threadIdx.x == 0) report(kBadRowLen, r, -1, n);
      return;
    }
    hi = n;
  } else {
    const int32_t p = lens[r];  // a position (attention, decode) or start position (compress)
    if (p < 0) {
      if (threadIdx.x == 0) report(kBadPosition, r, -1, p);
      return;
    }
    if (mode == kCheckWindow) {
      lo = p + 1 > window ? p + 1 - window : 0;
      hi = p + 1;
    } else if (mode == kCheckHca) {
      hi = (p + 1) / ratio;
    } else if (mode == kCheckCompress) {
      const int64_t n = cu_rows[r + 1] - cu_rows[r];
      if (n < 0) {
        if (threadIdx.x == 0) report(kBadRowLen, r, -1, (int32_t)n);
        return;
      }
      lo = p / ratio;
      hi = (p + n) / ratio;
    } else {  // kCheckDecode: the entry a decode token completes (if any), in the c4 table
      lo = (p + 1) / ratio - 1;
      hi = (p + 1) % ratio == 0 ? lo + 1 : lo;
      if (lo < 0) lo = hi = 0;
    }
  }
  if (hi <= lo) return;
  if (s < 0) {
    if (threadIdx.x == 0) report(kBadSequence, r, -1, s);
    return;
  }
  const int64_t p0 = lo / page_size, p1 = (hi + page_size - 1) / page_size;
  if (p1 > pt_stride) {
    if (threadIdx.x == 0) report(kBadTableWidth, r, (int32_t)(p1 - 1), pt_stride);
    return;
  }
  for (int64_t pg = p0 + threadIdx.x; pg < p1; pg += blockDim.x) {
    const int32_t id = pt[(int64_t)s * pt_stride + pg];
    if (id < 0 || id >= num_pages) report(kBadPage, r, (int32_t)pg, id);
  }
}

// Selected slots (R rows of k): each -1 or in [0, limit).
__global__ void __launch_bounds__(256)
check_idx_kernel(int64_t n, int k, const int32_t* __restrict__ idx, int64_t limit, int32_t code) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t v = idx[i];
    if (v < -1 || v >= limit) report(code, (int32_t)(i / k), (int32_t)(i % k), v);
  }
}

std::once_flag g_env_once;
std::atomic<int> g_debug{0};

void read_env() {
  const char* e = getenv("CSA_DEBUG");
  g_debug.store((e && e[0] && e[0] != '0') ? 1 : 0);
}

constexpr int kMaxDevices = 64;
std::mutex g_rec_mu;
int32_t* g_rec_ptr[kMaxDevices] = {};

int32_t* record_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_rec_mu);
  if (!g_rec_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_record)) != hipSuccess) return nullptr;
    g_rec_ptr[dev] = static_cast<int32_t*>(p);
  }
  return g_rec_ptr[dev];
}

const char* code_text(int32_t c) {
  switch (c) {
    case kBadRowLen: return "row length outside [0, capacity]";
    case kBadPosition: return "negative position";
    case kBadSequence: return "negative sequence index";
    case kBadTableWidth: return "entries past the page-table row (page index, row width)";
    case kBadPage: return "page id outside [0, num_pages)";
    case kBadSlot: return "selected slot outside [-1, pool slots)";
    case kBadEntry: return "selected entry outside [-1, max_entries)";
  }
  return "unknown violation";
}

}  // namespace

bool debug_on() {
  std::call_once(g_env_once, read_env);
  return g_debug.load() != 0;
}

void set_debug(int on) {
  std::call_once(g_env_once, read_env);
  g_debug.store(on ? 1 : 0);
}

DebugCheck::DebugCheck(const char* entry, hipStream_t s) : entry_(entry), s_(s) {
  rec_ = record_for_current_device();
  if (!rec_) {
    err_ = hipErrorInvalidSymbol;
    return;
  }
  hipLaunchKernelGGL(record_clear_kernel, dim3(1), dim3(64), 0, s_, rec_);
  err_ = hipGetLastError();
}

void DebugCheck::rows(int mode, int R, const int32_t* row_seq, const int32_t* lens, int64_t cap,
                      int ratio, int window, const int32_t* cu_rows, const int32_t* pt,
                      int pt_stride, int page_size, int64_t num_pages) {
  if (err_ != hipSuccess || R <= 0) return;
  hipLaunchKernelGGL(check_rows_kernel, dim3(R), dim3(256), 0, s_, mode, R, row_seq, lens, cap,
                     ratio, window, cu_rows, pt, pt_stride, page_size, num_pages);
  err_ = hipGetLastError();
}

void DebugCheck::idx(int64_t n, int k, const int32_t* v, int64_t limit, int32_t code) {
  if (err_ != hipSuccess || n <= 0) return;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(check_idx_kernel, dim3((unsigned)blocks), dim3(256), 0, s_, n, k, v, limit,
                     code);
  err_ = hipGetLastError();
}

csa_status DebugCheck::result() {
  if (err_ != hipSuccess) return CSA_ERR_HIP;
  int32_t h[4] = {0, 0, 0, 0};
  if (hipMemcpyAsync(h, rec_, sizeof(h), hipMemcpyDeviceToHost, s_) != hipSuccess ||
      hipStreamSynchronize(s_) != hipSuccess)
    return CSA_ERR_HIP;
  if (h[0] == 0) return CSA_OK;
  fprintf(stderr, "csa debug: %s: %s (row %d, index %d, value %d)\n", entry_, code_text(h[0]),
          h[1], h[2], h[3]);
  return CSA_ERR_BOUNDS;
}

}  // namespace csa
