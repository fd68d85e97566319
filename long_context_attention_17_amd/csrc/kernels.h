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

// Position of query row r: pos[r] (decode), or t0 + r (prefill rows of one sequence).
struct RowPos {
  const int32_t* pos;
  int t0;
  __device__ __forceinline__ int operator()(int r) const { return pos ? pos[r] : t0 + r; }
};

// Scores of every eligible block.  With ws_long (the multi-workgroup top-k state,
// used when the rows are long) the per-row key histograms are also cleared (unless
// state_zeroed: the caller cleared the kTopkRowWords words per row already) and filled.
constexpr int kTopkRowWords = 4096 + 4;   // per-row long top-k state: histogram bins, then 4 counters
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
  int split_items;     // 0: one split per row (direct epilogue); else the minimum split length
  int split_div;       // a row of n items is split into chunks of max(split_items, ceil64(n / split_div))
  int max_splits;      // splits per row the workspace holds (never exceeded)
  float* part_o;       // [rows, max_splits, n_heads, D]
  float* part_ml;      // [rows, max_splits, n_heads, 2]
  int part_acc;        // 1: part_o is in the MFMA kernel's accumulator layout (see attend_combine_kernel)
  int part_bf16;       // 1 (accumulator layout, bf16 output): part_o holds bf16 values, same element offsets
  uint16_t* q_prep;    // nullptr, or bf16 [rows, n_heads, D]: queries normalized, rotated and scaled
                       // once per row by a prep kernel (split rows of the MFMA path)
};

// Decode split plan: chunks of at least kDecodeSplitItems items, at most
// kDecodeMaxSplits chunks per row (a function of the row alone).
constexpr int kDecodeSplitItems = 256;
constexpr int kDecodeMaxSplits = 16;

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
