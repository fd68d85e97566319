// Internal launcher declarations of the CSA / HCA kernels.
#pragma once
#include <hip/hip_runtime.h>

#include "common.h"

namespace ca {

// Rows Ca.. hold positions t0 .. t0+L-1; emits the entries whose pooling window lies
// inside them (see ca_compress_prefill).
hipError_t launch_compress_prefill(const CacheView& cv, int seq, const ca_compress_params& p, const void* Ca,
                                   const void* Za, const void* Cb, const void* Zb, const float* Ba,
                                   const float* Bb, const float* gain, int64_t L, int64_t t0, hipStream_t st);
hipError_t launch_compress_decode(const CacheView& cv, const ca_compress_params& p, const void* new_rows,
                                  const int32_t* pos, int B, float* tail, const float* Ba, const float* Bb,
                                  const float* gain, hipStream_t st);
hipError_t launch_store_entries(const CacheView& cv, int seq, int64_t first, int64_t n, const float* src,
                                const float* gain, float eps, int apply_rope, double base, int pos_stride,
                                hipStream_t st);
hipError_t launch_window_append(const ca_window_params& p, const void* raw, const float* gain, const int32_t* pos,
                                const int32_t* seq, int T, void* window, int W, int S, hipStream_t st);

// The fused decode append (ca_decode_append): the window append of every row b
// (sequence b) plus one or two compressor steps, in one launch.
struct DecodeWindowJob {
  int D, R, in_fmt, win_fmt;
  const void* raw;
  const float* gain;
  void* window;
  int W, S;
  float eps;
  double base;
};
struct DecodeEntryJob {
  CacheView cv;
  int m, overlap, in_fmt, apply_rope;
  const void* new_rows;
  float* tail;
  const float *Ba, *Bb, *gain;   // gain: nullptr unless the epilogue normalizes
  float eps;
  double base;
};

// Device status bits (ca_status_bits in the header): OR-ed into a caller's status word.
__device__ __forceinline__ void raise_status(int32_t* status, int32_t bits) {
  if (status != nullptr) atomicOr(status, bits);
}

// Position of query row r: pos[r] (decode), or t0 + r (prefill rows of one sequence).
// A decode position outside [0, max_pos] is out of contract: it reads as -1 (a row
// with no eligible entries) and raises CA_STATUS_POS_RANGE in *status.
struct RowPos {
  const int32_t* pos;
  int t0;
  int max_pos;
  int32_t* status;
  __device__ __forceinline__ int operator()(int r) const { return of(r, pos != nullptr ? pos[r] : 0); }
  // The same from row r's pos word as already loaded (raw; ignored when pos == nullptr).
  __device__ __forceinline__ int of(int r, int raw) const {
    if (pos == nullptr) return t0 + r;
    if (raw < 0 || raw > max_pos) {
      raise_status(status, CA_STATUS_POS_RANGE);
      return -1;
    }
    return raw;
  }
};

// Scores of every eligible block.  With ws_long (the multi-workgroup top-k state,
// used when the rows are long) the per-row key histograms are also cleared (unless
// state_zeroed: the caller cleared the kTopkRowWords words per row already) and filled.
constexpr int kTopkRowWords = 4096 + 4 + 64;   // per-row long top-k state: histogram bins, 4 counters, 64 coarse bins
hipError_t launch_index_scores(const CacheView& cv, const ca_index_params& p, const void* qI, const float* w,
                               RowPos pos, int seq_fixed, int n_rows, int64_t max_pos, float* scores,
                               int64_t stride, void* ws_long, hipStream_t st, bool state_zeroed = false);
// Top-k over score rows.  With ws_long (topk_long_workspace bytes) and rows longer than
// one workgroup's LDS, the multi-workgroup histogram / gather / resolve path runs.
size_t topk_long_workspace(int n_rows, int64_t stride);
bool topk_use_long(int64_t stride, int k);
hipError_t launch_topk(const float* scores, int64_t stride, RowPos pos, int m, int k, int n_rows,
                       int32_t* out_idx, int32_t* out_cnt, float* out_score, void* ws_long, hipStream_t st);

// Everything an attention launch needs (CSA or HCA, prefill or decode).
struct AttendArgs {
  const void* q;
  const float* q_gain;
  int q_fmt, n_heads, D, R, n_win;
  float scale_log2;  // logit scale * log2(e)
  float eps;
  double base;
  double rope_step;    // base^(-2/R): the rotary frequency of pair p is rope_step^p
  const int32_t* pos;  // nullptr: position == t0 + row (prefill)
  int t0;              // position of row 0 when pos == nullptr
  int seq_fixed;       // >= 0: every row is this cache sequence (prefill); < 0: row r is sequence r
  int n_rows;
  CacheView kv;
  int mode;            // 0: CSA list idx/cnt, 1: HCA dense
  int ratio;
  const int32_t* idx;
  const int32_t* cnt;
  int k;
  const void* win;
  int win_fmt, W;
  const float* sink;
  void* out;
  int out_fmt;
  float* lse;
  int max_pos;         // decode: the caller's bound on pos[r]; rows beyond it (or negative) are
                       // out of contract (no items, zero output, CA_STATUS_POS_RANGE raised)
  int32_t* status;     // optional device status word (CA_STATUS_* bits are OR-ed in)
  int split_min;       // 0: one split per row (direct epilogue); else the minimum split length
  int split_div;       // chunks a row is split into at least (when long enough), see split_plan_len
  int split_cap;       // the longest chunk (one MFMA workgroup's item table)
  int max_splits;      // splits per row the workspace holds (never exceeded)
  float* part_o;       // [rows, max_splits, n_heads, D]
  float* part_ml;      // [rows, max_splits, n_heads, 2]
  int part_acc;        // 1: part_o is in the MFMA kernel's accumulator layout (see attend_combine_kernel)
  int part_bf16;       // 1 (bf16 output): part_o holds bf16 values at the same element offsets
  int dense_units;     // 1: the MFMA kernel numbers a decode launch's real units densely (set by launch_attend)
  uint16_t* q_prep;    // nullptr, or bf16 [rows, n_heads, D]: queries times gain and logit scale,
                       // rotated, once per row by a prep kernel (split rows of the MFMA path)
  float* q_inv;        // with q_prep: [rows, n_heads], each query row's RMSNorm factor 1 / rms,
                       // which scales its logits (q_prep holds the row without it)
};

// Split plan of a row of `total` items, a function of the row alone (so a decode
// row's accumulation order does not depend on the batch): d = max(split_div,
// ceil(total / split_cap)) chunks of ceil64(total / d) items, but never shorter
// than split_min.  A chunk never exceeds split_cap (a multiple of 64), and a row
// of at most max_items items has at most plan_max_splits(max_items) chunks.
constexpr int kDecodeSplitItems = 256;   // decode: split_min
constexpr int kDecodeMaxSplits = 16;     // decode: split_div

__host__ __device__ __forceinline__ int split_plan_len(int64_t total, int split_min, int split_div, int split_cap) {
  int64_t d = (total + split_cap - 1) / split_cap;
  d = d > split_div ? d : split_div;
  d = d > 0 ? d : 1;
  int64_t len = (total + d - 1) / d;
  len = (len + 63) & ~(int64_t)63;
  return (int)(len > split_min ? len : split_min);
}
// The same plan in 32-bit arithmetic for the kernels (a row's item count stays below
// 2^31 - split_cap; 64-bit divisions are long instruction sequences on the GPU).
__device__ __forceinline__ int split_plan_len32(int total, int split_min, int split_div, int split_cap) {
  int d = (total + split_cap - 1) / split_cap;
  d = d > split_div ? d : split_div;
  d = d > 0 ? d : 1;
  const int len = ((total + d - 1) / d + 63) & ~63;
  return len > split_min ? len : split_min;
}
__device__ __forceinline__ int split_plan_count32(int total, int split_min, int split_div, int split_cap) {
  const int len = split_plan_len32(total, split_min, split_div, split_cap);
  const int n = (total + len - 1) / len;
  return n > 0 ? n : 1;
}
__host__ __device__ __forceinline__ int split_plan_count(int64_t total, int split_min, int split_div, int split_cap) {
  const int64_t len = split_plan_len(total, split_min, split_div, split_cap);
  const int64_t n = (total + len - 1) / len;
  return (int)(n > 0 ? n : 1);
}
__host__ __device__ __forceinline__ int plan_max_splits(int64_t max_items, int split_min, int split_div,
                                                        int split_cap) {
  const int64_t by_len = (max_items + split_min - 1) / split_min;
  int64_t d = (max_items + split_cap - 1) / split_cap;
  d = d > split_div ? d : split_div;
  const int64_t n = by_len < d ? by_len : d;
  return (int)(n > 0 ? n : 1);
}

bool attend_mfma_supported(const AttendArgs& a);
int attend_mfma_max_items();  // items one MFMA workgroup handles without splitting
// q_prepared: split rows' queries are already in a.q_prep (no query-prep launch).
hipError_t launch_attend(const AttendArgs& a, hipStream_t st, bool q_prepared = false);

// The front of a decode step (ca_decode_append, ca_*_decode_step): the window append
// of every row b (sequence b) and one or two compressor steps, plus optionally the
// query preparation of qa (when qa->q_prep != nullptr) and the clearing of
// zero_words words per row at zero, in one launch.
hipError_t launch_decode_front(const DecodeWindowJob& wj, const DecodeEntryJob* jobs, int n_jobs,
                               const int32_t* pos, int B, const AttendArgs* qa, uint32_t* zero, int zero_words,
                               hipStream_t st);
hipError_t launch_decode_append(const DecodeWindowJob& wj, const DecodeEntryJob* jobs, int n_jobs,
                                const int32_t* pos, int B, hipStream_t st);

// C_b = A_b W_b^T for b < batch (bf16 operands, both K-contiguous; fp32 accumulation).
// A_b [M, K]: row stride lda, batch stride a_batch (elements).  Up to two N segments
// share A, each with its own W_b [N, K] (ldw, w_batch) and C_b [M, N] (ldc, c_batch,
// bf16 or fp32).  K % 64 == 0; A, W 16-byte aligned with lda, ldw, a_batch, w_batch
// multiples of 8.  part: fp32 workspace of part_floats floats (set by gemm_plan) for the
// K splits, nullptr when that is 0.
struct GemmSeg {
  const void* W;
  void* C;
  int N, c_f32;
  int64_t ldw, ldc, w_batch, c_batch;
  int n_tiles;          // set by gemm_plan
  int64_t part_off;     // set by gemm_plan
};
struct GemmArgs {
  const void* A;
  int64_t lda, a_batch;
  int M, K, batch, n_seg;
  GemmSeg seg[2];
  float* part;
  // set by gemm_plan
  int tile_m, tile_n;   // workgroup tile: 32 x 128, 128 x 128 or 256 x 256
  int m_tiles, n_tiles, k_tiles, k_splits;
  int64_t part_floats, grid_blocks;
};
void gemm_plan(GemmArgs& g);
hipError_t launch_gemm(GemmArgs g, hipStream_t st);

// One sequence's decode state as parts copied between their live storage and a flat
// buffer (state.hip).  A part is n_items items of item_bytes (a multiple of 16) each,
// contiguous in live storage, or (page_table != nullptr) one page each, found through
// the sequence's page-table row.
struct StatePart {
  uint8_t* live;
  const int32_t* page_table;   // the sequence's row, or nullptr
  int64_t n_pages;
  int64_t item_bytes, n_items, chunks_per_item;   // chunks of 4 KB
  int64_t flat_offset;
};
struct StatePlan {
  uint8_t* buffer;
  int n_parts;
  StatePart part[5];
};
hipError_t launch_state_copy(const StatePlan& p, int to_buffer, hipStream_t st);

// Launch timing of the timed kernels (ids: ca_timed_kernel): the start / stop
// events for the next launch of `kernel` on `st`, or false (both null) when it
// is not being timed.  CA_LAUNCH launches through hipExtLaunchKernelGGL with
// the events when they are set, else with hipLaunchKernelGGL.
bool timer_events(int kernel, hipStream_t st, hipEvent_t* start, hipEvent_t* stop);
#define CA_LAUNCH(kernel, grid, block, smem, st, ev0, ev1, ...)                       \
  do {                                                                              \
    if (ev0 != nullptr)                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, smem, st, ev0, ev1, 0, __VA_ARGS__); \
    else                                                                            \
      hipLaunchKernelGGL(kernel, grid, block, smem, st, __VA_ARGS__);               \
  } while (0)

}  // namespace ca
