// C ABI of the CSA / HCA library: host-side validation, workspace layout and
// dispatch to the kernels.  No allocation, no host synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/csahca.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return CA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_act(int f) { return f == CA_F32 || f == CA_BF16; }

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// Validate a cache descriptor and build its device view.
int make_view(const ca_cache* c, ca::CacheView* v, const char* what) {
  if (c == nullptr) return fail(CA_ERR_ARG, "%s: cache descriptor is NULL", what);
  if (c->format < CA_F32 || c->format > CA_FP4) return fail(CA_ERR_DTYPE, "%s: unknown cache format %d", what, c->format);
  if (c->dim <= 0 || c->dim > 1024) return fail(CA_ERR_UNSUPPORTED, "%s: dim %d outside 1..1024", what, c->dim);
  if (c->rope_dim < 0 || c->rope_dim > c->dim || (c->rope_dim & 1))
    return fail(CA_ERR_ARG, "%s: rope_dim %d must be even and <= dim", what, c->rope_dim);
  if (c->format == CA_FP8MIX && ((c->dim - c->rope_dim) % 64 != 0))
    return fail(CA_ERR_UNSUPPORTED, "%s: fp8-mixed records need (dim - rope_dim) %% 64 == 0", what);
  if ((c->format == CA_E4M3 || c->format == CA_FP4) && c->rope_dim != 0)
    return fail(CA_ERR_ARG, "%s: indexer pools have rope_dim 0", what);
  if (c->format == CA_FP4 && c->dim % 32 != 0)
    return fail(CA_ERR_UNSUPPORTED, "%s: FP4 pools need dim %% 32 == 0 (one scale per 32 channels)", what);
  if (!pow2(c->page_size)) return fail(CA_ERR_ARG, "%s: page_size %d must be a power of two", what, c->page_size);
  if (c->n_pages < 0 || c->n_seqs < 0 || c->max_pages < 0) return fail(CA_ERR_ARG, "%s: negative sizes", what);
  if (c->n_pages > 0 && c->pool == nullptr) return fail(CA_ERR_ARG, "%s: pool is NULL", what);
  if (c->n_seqs > 0 && c->max_pages > 0 && c->page_table == nullptr) return fail(CA_ERR_ARG, "%s: page_table is NULL", what);
  v->pool = (uint8_t*)c->pool;
  v->page_table = c->page_table;
  v->n_pages = c->n_pages;
  v->page_bytes = ca::page_bytes(c->format, c->dim, c->rope_dim, c->page_size);
  v->stride = ca::record_stride(c->format, c->dim, c->rope_dim);
  v->max_pages = c->max_pages;
  v->page_shift = ilog2(c->page_size);
  v->fmt = c->format;
  v->dim = c->dim;
  v->rope = c->rope_dim;
  return CA_OK;
}

hipStream_t S(void* s) { return (hipStream_t)s; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int64_t score_stride(int64_t max_pos, int ratio) {
  int64_t ne = max_pos / ratio;
  if (ne < 1) ne = 1;
  return (ne + 63) / 64 * 64;
}

// Items of the longest row of an attention call: its entries (k for CSA, the
// eligible entries at max_pos for HCA) plus the window.
int64_t max_items_of(int64_t max_pos, int n_win, int k, int ratio) {
  return (k > 0 ? (int64_t)k : max_pos / ratio) + n_win;
}

// The decode split plan (minimum chunk, chunks) of a call's rows: a constant of the call,
// never of the batch.
void decode_plan_of(int n_heads, int D, int R, int* split_min, int* split_div) {
  (void)n_heads;
  (void)D;
  (void)R;
  *split_min = ca::kDecodeSplitItems;
  *split_div = ca::kDecodeMaxSplits;
}

// Splits per row the decode plan can make (an upper bound for the prefill plan too,
// whose chunks are never shorter than the decode plan's for the same row).
int max_splits_for(const ca_attend_params* p, int64_t max_pos, int k, int ratio) {
  int mn, dv;
  decode_plan_of(p->n_heads, p->dim, p->rope_dim, &mn, &dv);
  return ca::plan_max_splits(max_items_of(max_pos, p->n_win, k, ratio), mn, dv, ca::attend_mfma_max_items());
}

}  // namespace

extern "C" {

const char* ca_last_error(void) { return g_err; }

int64_t ca_record_stride(int32_t format, int32_t dim, int32_t rope_dim) {
  if (format < CA_F32 || format > CA_FP4 || dim <= 0 || (format == CA_FP4 && dim % 32 != 0)) return -1;
  return ca::record_stride(format, dim, rope_dim);
}

int64_t ca_page_bytes(int32_t format, int32_t dim, int32_t rope_dim, int32_t page_size) {
  if (format < CA_F32 || format > CA_FP4 || dim <= 0 || page_size <= 0 || (format == CA_FP4 && dim % 32 != 0)) return -1;
  return ca::page_bytes(format, dim, rope_dim, page_size);
}

int ca_store_entries(const ca_cache* cache, int32_t seq, int64_t first, int64_t n, const float* src,
                     const float* gain, float eps, int32_t apply_rope, double rope_base, int32_t pos_stride,
                     void* stream) {
  ca::CacheView cv;
  if (int e = make_view(cache, &cv, "ca_store_entries")) return e;
  if (n < 0 || first < 0) return fail(CA_ERR_ARG, "ca_store_entries: negative first/n");
  if (n > 0 && src == nullptr) return fail(CA_ERR_ARG, "ca_store_entries: src is NULL");
  if (seq < 0 || seq >= cache->n_seqs) return fail(CA_ERR_ARG, "ca_store_entries: seq %d out of range", seq);
  if (first + n > (int64_t)cache->max_pages * cache->page_size)
    return fail(CA_ERR_ARG, "ca_store_entries: entries beyond the page table");
  if (n > 0x7FFFFFFF) return fail(CA_ERR_UNSUPPORTED, "ca_store_entries: n too large");
  return hip_status(ca::launch_store_entries(cv, seq, first, n, src, gain, eps, apply_rope, rope_base, pos_stride,
                                             S(stream)),
                    "ca_store_entries");
}

static int check_compress(const ca_compress_params* p, const ca_cache* cache, ca::CacheView* cv, const char* w) {
  if (p == nullptr) return fail(CA_ERR_ARG, "%s: params NULL", w);
  if (int e = make_view(cache, cv, w)) return e;
  if (p->ratio <= 0) return fail(CA_ERR_ARG, "%s: ratio must be positive", w);
  if (p->overlap != 0 && p->overlap != 1) return fail(CA_ERR_ARG, "%s: overlap must be 0 or 1", w);
  if (!is_act(p->in_format)) return fail(CA_ERR_DTYPE, "%s: in_format must be F32 or BF16", w);
  return CA_OK;
}

int ca_compress_prefill(const ca_compress_params* p, const void* Ca, const void* Za, const void* Cb,
                        const void* Zb, const float* Ba, const float* Bb, const float* gain, int64_t L, int64_t t0,
                        int32_t seq, const ca_cache* cache, void* stream) {
  ca::CacheView cv;
  if (int e = check_compress(p, cache, &cv, "ca_compress_prefill")) return e;
  if (L < 0 || t0 < 0 || t0 + L > 0x7FFFFFFF) return fail(CA_ERR_ARG, "ca_compress_prefill: bad L / t0");
  if ((t0 + L) / p->ratio <= ca::compress_first_entry(p->ratio, p->overlap, t0)) return ok();
  if (!Ca || !Za || !Ba) return fail(CA_ERR_ARG, "ca_compress_prefill: Ca/Za/Ba NULL");
  if (p->overlap && (!Cb || !Zb || !Bb)) return fail(CA_ERR_ARG, "ca_compress_prefill: Cb/Zb/Bb NULL with overlap");
  if (p->apply_norm && !gain) return fail(CA_ERR_ARG, "ca_compress_prefill: gain NULL with apply_norm");
  if (seq < 0 || seq >= cache->n_seqs) return fail(CA_ERR_ARG, "ca_compress_prefill: seq out of range");
  if ((t0 + L) / p->ratio > (int64_t)cache->max_pages * cache->page_size)
    return fail(CA_ERR_ARG, "ca_compress_prefill: page table holds fewer than (t0+L)/ratio entries");
  return hip_status(ca::launch_compress_prefill(cv, seq, *p, Ca, Za, Cb, Zb, Ba, Bb, gain, L, t0, S(stream)),
                    "ca_compress_prefill");
}

int ca_compress_decode(const ca_compress_params* p, const void* new_rows, const int32_t* pos, int32_t B,
                       float* tail, const float* Ba, const float* Bb, const float* gain, const ca_cache* cache,
                       void* stream) {
  ca::CacheView cv;
  if (int e = check_compress(p, cache, &cv, "ca_compress_decode")) return e;
  if (B < 0) return fail(CA_ERR_ARG, "ca_compress_decode: negative B");
  if (B == 0) return ok();
  if (!new_rows || !pos || !tail || !Ba) return fail(CA_ERR_ARG, "ca_compress_decode: NULL argument");
  if (p->overlap && !Bb) return fail(CA_ERR_ARG, "ca_compress_decode: Bb NULL with overlap");
  if (p->apply_norm && !gain) return fail(CA_ERR_ARG, "ca_compress_decode: gain NULL with apply_norm");
  if (B > cache->n_seqs) return fail(CA_ERR_ARG, "ca_compress_decode: B exceeds the page table rows");
  return hip_status(ca::launch_compress_decode(cv, *p, new_rows, pos, B, tail, Ba, Bb, gain, S(stream)),
                    "ca_compress_decode");
}

int ca_window_append(const ca_window_params* p, const void* kv_raw, const float* gain, const int32_t* pos,
                     const int32_t* seq, int32_t T, void* window, int32_t W, int32_t S_, void* stream) {
  if (p == nullptr) return fail(CA_ERR_ARG, "ca_window_append: params NULL");
  if (p->dim <= 0 || p->dim > 1024) return fail(CA_ERR_UNSUPPORTED, "ca_window_append: dim outside 1..1024");
  if (p->rope_dim < 0 || p->rope_dim > p->dim || (p->rope_dim & 1)) return fail(CA_ERR_ARG, "ca_window_append: bad rope_dim");
  if (!is_act(p->in_format) || !is_act(p->win_format)) return fail(CA_ERR_DTYPE, "ca_window_append: formats must be F32/BF16");
  if (T < 0 || W <= 0 || S_ <= 0) return fail(CA_ERR_ARG, "ca_window_append: bad T/W/S");
  if (T == 0) return ok();
  if (!kv_raw || !gain || !window) return fail(CA_ERR_ARG, "ca_window_append: NULL argument");
  return hip_status(ca::launch_window_append(*p, kv_raw, gain, pos, seq, T, window, W, S_, S(stream)),
                    "ca_window_append");
}

// Validates a decode append (ca_decode_append's checks) and fills its launch jobs.
static int append_plan(const ca_window_params* wp, const void* kv_raw, const float* w_gain, const int32_t* pos,
                       int32_t B, void* window, int32_t W, int32_t S_, const ca_decode_entry_job* jobs,
                       int32_t n_jobs, ca::DecodeWindowJob* wjob, ca::DecodeEntryJob* ej, const char* what) {
  if (wp == nullptr) return fail(CA_ERR_ARG, "%s: window params NULL", what);
  if (wp->dim <= 0 || wp->dim > 1024) return fail(CA_ERR_UNSUPPORTED, "%s: window dim outside 1..1024", what);
  if (wp->rope_dim < 0 || wp->rope_dim > wp->dim || (wp->rope_dim & 1)) return fail(CA_ERR_ARG, "%s: bad rope_dim", what);
  if (!is_act(wp->in_format) || !is_act(wp->win_format)) return fail(CA_ERR_DTYPE, "%s: formats must be F32/BF16", what);
  if (n_jobs < 1 || n_jobs > 2 || jobs == nullptr) return fail(CA_ERR_ARG, "%s: n_jobs must be 1 or 2", what);
  if (B < 0 || W <= 0 || S_ < B) return fail(CA_ERR_ARG, "%s: bad B/W/S (S must hold every row's sequence)", what);
  for (int q = 0; q < n_jobs; ++q) {
    const ca_decode_entry_job& j = jobs[q];
    if (int e = check_compress(&j.params, j.cache, &ej[q].cv, what)) return e;
    if (B > 0 && (!j.new_rows || !j.tail || !j.Ba)) return fail(CA_ERR_ARG, "%s: job %d: NULL argument", what, q);
    if (B > 0 && j.params.overlap && !j.Bb) return fail(CA_ERR_ARG, "%s: job %d: Bb NULL with overlap", what, q);
    if (B > 0 && j.params.apply_norm && !j.gain) return fail(CA_ERR_ARG, "%s: job %d: gain NULL with apply_norm", what, q);
    if (B > j.cache->n_seqs) return fail(CA_ERR_ARG, "%s: job %d: B exceeds the page table rows", what, q);
    ej[q].m = j.params.ratio;
    ej[q].overlap = j.params.overlap;
    ej[q].in_fmt = j.params.in_format;
    ej[q].apply_rope = j.params.apply_rope;
    ej[q].new_rows = j.new_rows;
    ej[q].tail = j.tail;
    ej[q].Ba = j.Ba;
    ej[q].Bb = j.Bb;
    ej[q].gain = j.params.apply_norm ? j.gain : nullptr;
    ej[q].eps = j.params.eps;
    ej[q].base = j.params.rope_base;
  }
  if (B == 0) return CA_OK;
  if (!kv_raw || !w_gain || !window || !pos) return fail(CA_ERR_ARG, "%s: NULL argument", what);
  *wjob = ca::DecodeWindowJob{wp->dim, wp->rope_dim, wp->in_format, wp->win_format, kv_raw, w_gain, window, W, S_,
                              wp->eps, wp->rope_base};
  return CA_OK;
}

int ca_decode_append(const ca_window_params* wp, const void* kv_raw, const float* w_gain, const int32_t* pos,
                     int32_t B, void* window, int32_t W, int32_t S_, const ca_decode_entry_job* jobs, int32_t n_jobs,
                     void* stream) {
  const char* what = "ca_decode_append";
  ca::DecodeWindowJob wj;
  ca::DecodeEntryJob ej[2];
  if (int e = append_plan(wp, kv_raw, w_gain, pos, B, window, W, S_, jobs, n_jobs, &wj, ej, what)) return e;
  if (B == 0) return ok();
  return hip_status(ca::launch_decode_append(wj, ej, n_jobs, pos, B, S(stream)), what);
}

// ------------------------------------------------------------------ indexer
// Workspace: the score rows, then (for long rows) the multi-workgroup top-k state.
size_t ca_index_topk_workspace(const ca_index_params* p, int32_t n_rows, int64_t max_pos) {
  if (p == nullptr || p->ratio <= 0 || n_rows <= 0 || max_pos < 0) return 0;
  int64_t stride = score_stride(max_pos, p->ratio);
  size_t bytes = align256((size_t)n_rows * stride * sizeof(float));
  if (ca::topk_use_long(stride, p->k)) bytes += align256(ca::topk_long_workspace(n_rows, stride));
  return bytes;
}

// A validated indexer call, ready to launch (n_rows == 0: nothing to do).
struct IndexPlan {
  ca::CacheView cv;
  ca_index_params p;
  const void* qI;
  const float* w;
  ca::RowPos rp;
  int seq_fixed, n_rows;
  int64_t max_pos;
  float* scores;
  int64_t stride;
  void* ws_long;
  int32_t *out_idx, *out_cnt;
  float* out_score;
};

static hipError_t launch_index_plan(const IndexPlan& ip, hipStream_t st, bool state_zeroed) {
  if (ip.n_rows == 0) return hipSuccess;
  hipError_t e = ca::launch_index_scores(ip.cv, ip.p, ip.qI, ip.w, ip.rp, ip.seq_fixed, ip.n_rows, ip.max_pos,
                                         ip.scores, ip.stride, ip.ws_long, st, state_zeroed);
  if (e != hipSuccess) return e;
  return ca::launch_topk(ip.scores, ip.stride, ip.rp, ip.p.ratio, ip.p.k, ip.n_rows, ip.out_idx, ip.out_cnt,
                         ip.out_score, ip.ws_long, st);
}

// Validates an indexer call; launches it, or (plan != nullptr) only describes it.
static int index_common(const ca_index_params* p, const void* qI, const float* w, const int32_t* pos, int64_t t0,
                        int seq_fixed,
                        int64_t n_rows, int64_t max_pos, const ca_cache* idx_cache, int32_t* out_idx,
                        int32_t* out_cnt, float* out_score, float* all_scores, int64_t all_stride, void* ws,
                        size_t ws_bytes, void* stream, const char* what, IndexPlan* plan = nullptr) {
  if (plan) plan->n_rows = 0;
  if (p == nullptr) return fail(CA_ERR_ARG, "%s: params NULL", what);
  ca::CacheView cv;
  if (int e = make_view(idx_cache, &cv, what)) return e;
  if (idx_cache->format != CA_F32 && idx_cache->format != CA_E4M3 && idx_cache->format != CA_FP4)
    return fail(CA_ERR_DTYPE, "%s: indexer pool must be F32, E4M3 or FP4", what);
  if (p->dim != idx_cache->dim) return fail(CA_ERR_ARG, "%s: params dim %d != cache dim %d", what, p->dim, idx_cache->dim);
  if (p->n_heads <= 0 || p->dim <= 0 || p->ratio <= 0 || p->k <= 0) return fail(CA_ERR_ARG, "%s: bad params", what);
  if ((int64_t)p->n_heads * p->dim > 16384) return fail(CA_ERR_UNSUPPORTED, "%s: n_heads*dim > 16384", what);
  if (!is_act(p->q_format)) return fail(CA_ERR_DTYPE, "%s: q_format must be F32/BF16", what);
  if (p->q_quant != 0 && !(p->q_quant == CA_FP4 && idx_cache->format == CA_FP4))
    return fail(CA_ERR_ARG, "%s: q_quant must be 0, or CA_FP4 with an FP4 indexer pool", what);
  if (n_rows < 0 || n_rows > 0x7FFFFFFF) return fail(CA_ERR_ARG, "%s: bad row count", what);
  if (max_pos > 0x7FFFFFFF) return fail(CA_ERR_ARG, "%s: max_pos beyond 2^31 - 1", what);
  if (n_rows == 0) return ok();
  if (!qI || !w || !out_idx || !out_cnt) return fail(CA_ERR_ARG, "%s: NULL argument", what);
  if (max_pos / p->ratio > (int64_t)idx_cache->max_pages * idx_cache->page_size)
    return fail(CA_ERR_ARG, "%s: page table holds fewer entries than floor(max_pos/ratio)", what);
  float* scores;
  int64_t stride;
  void* ws_long = nullptr;
  if (all_scores != nullptr) {
    if (all_stride < max_pos / p->ratio || all_stride < 1) return fail(CA_ERR_ARG, "%s: all_scores_stride too small", what);
    scores = all_scores;
    stride = all_stride;
    if (ca::topk_use_long(stride, p->k)) {
      size_t need = align256(ca::topk_long_workspace((int)n_rows, stride));
      if (ws != nullptr && ws_bytes >= need) ws_long = ws;
    }
  } else {
    size_t need = ca_index_topk_workspace(p, (int32_t)n_rows, max_pos);
    if (ws_bytes < need || (need > 0 && ws == nullptr))
      return fail(CA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", what, ws_bytes, need);
    scores = (float*)ws;
    stride = score_stride(max_pos, p->ratio);
    if (ca::topk_use_long(stride, p->k))
      ws_long = (char*)ws + align256((size_t)n_rows * stride * sizeof(float));
  }
  IndexPlan ip{cv, *p, qI, w, ca::RowPos{pos, (int)t0, (int)max_pos, p->status}, seq_fixed, (int)n_rows, max_pos,
               scores, stride, ws_long, out_idx, out_cnt, out_score};
  if (plan) {
    *plan = ip;
    return CA_OK;
  }
  return hip_status(launch_index_plan(ip, S(stream), false), what);
}

int ca_index_topk_prefill(const ca_index_params* p, const void* qI, const float* w, int64_t L, int64_t t0,
                          int32_t seq, const ca_cache* idx_cache, int32_t* out_idx, int32_t* out_cnt,
                          float* out_score, float* all_scores, int64_t all_scores_stride, void* ws, size_t ws_bytes,
                          void* stream) {
  if (idx_cache && (seq < 0 || seq >= idx_cache->n_seqs)) return fail(CA_ERR_ARG, "ca_index_topk_prefill: seq out of range");
  if (t0 < 0 || L < 0 || t0 + L > 0x7FFFFFFF) return fail(CA_ERR_ARG, "ca_index_topk_prefill: bad L / t0");
  return index_common(p, qI, w, nullptr, t0, seq, L, L > 0 ? t0 + L - 1 : 0, idx_cache, out_idx, out_cnt, out_score,
                      all_scores, all_scores_stride, ws, ws_bytes, stream, "ca_index_topk_prefill");
}

int ca_index_topk_decode(const ca_index_params* p, const void* qI, const float* w, const int32_t* pos,
                         int32_t B, int64_t max_pos, const ca_cache* idx_cache, int32_t* out_idx,
                         int32_t* out_cnt, float* out_score, float* all_scores, int64_t all_scores_stride,
                         void* ws, size_t ws_bytes, void* stream) {
  if (pos == nullptr && B > 0) return fail(CA_ERR_ARG, "ca_index_topk_decode: pos NULL");
  if (idx_cache && B > idx_cache->n_seqs) return fail(CA_ERR_ARG, "ca_index_topk_decode: B exceeds page table rows");
  if (max_pos < 0) return fail(CA_ERR_ARG, "ca_index_topk_decode: negative max_pos");
  return index_common(p, qI, w, pos, 0, -1, B, max_pos, idx_cache, out_idx, out_cnt, out_score, all_scores,
                      all_scores_stride, ws, ws_bytes, stream, "ca_index_topk_decode");
}

// ------------------------------------------------------------------ attention
// Bytes for the split partials (o, m, l) of every row: an upper bound for both decode
// and prefill (prefill needs them only for rows longer than one workgroup's item table).
size_t ca_attend_workspace(const ca_attend_params* p, int32_t n_rows, int64_t max_pos, int32_t k, int32_t ratio) {
  if (p == nullptr || n_rows <= 0 || ratio <= 0) return 0;
  size_t ms = (size_t)max_splits_for(p, max_pos, k, ratio);
  // partials are stored no finer than the output: bf16 for a bf16 output, else fp32
  const size_t esz = p->out_format == CA_BF16 ? 2 : sizeof(float);
  size_t po = (size_t)n_rows * ms * p->n_heads * p->dim * esz;
  size_t pm = (size_t)n_rows * ms * p->n_heads * 2 * sizeof(float);
  size_t pq = (size_t)n_rows * p->n_heads * p->dim * 2;   // prepared bf16 queries
  size_t pi = (size_t)n_rows * p->n_heads * sizeof(float);  // their RMSNorm factors
  return align256(po) + align256(pm) + align256(pq) + align256(pi);
}

// ------------------------------------------------------------------ decode state
static int state_plan(const ca_decode_state* st, int32_t seq, int64_t pos, void* buffer, ca::StatePlan* plan,
                      int64_t* total, const char* what) {
  if (st == nullptr) return fail(CA_ERR_ARG, "%s: state descriptor NULL", what);
  if (st->n_jobs < 1 || st->n_jobs > 2) return fail(CA_ERR_ARG, "%s: n_jobs must be 1 or 2", what);
  if (st->W <= 0 || st->S <= 0 || st->win_dim <= 0 || !is_act(st->win_format))
    return fail(CA_ERR_ARG, "%s: bad window shape or format", what);
  if (seq < 0 || seq >= st->S) return fail(CA_ERR_ARG, "%s: seq %d outside the window's %d rows", what, seq, st->S);
  if (pos < 0) return fail(CA_ERR_ARG, "%s: negative pos", what);
  if (st->window == nullptr) return fail(CA_ERR_ARG, "%s: window NULL", what);
  if (((uintptr_t)st->window | (uintptr_t)buffer | (uintptr_t)st->tail[0] | (uintptr_t)st->tail[1]) % 16)
    return fail(CA_ERR_ARG, "%s: window, tails and buffer must be 16-byte aligned", what);
  ca::StatePlan p{};
  p.buffer = (uint8_t*)buffer;
  int64_t off = 0;
  auto add = [&](uint8_t* live, const int32_t* pt, int64_t n_pages, int64_t item_bytes, int64_t n_items) {
    ca::StatePart& q = p.part[p.n_parts++];
    q.live = live;
    q.page_table = pt;
    q.n_pages = n_pages;
    q.item_bytes = item_bytes;
    q.n_items = n_items;
    q.chunks_per_item = (item_bytes + 4095) / 4096;
    q.flat_offset = off;
    off = align256(off + item_bytes * n_items);
  };
  const int64_t esz = st->win_format == CA_F32 ? 4 : 2;
  const int64_t wrow = (int64_t)st->W * st->win_dim * esz;
  if (wrow % 16) return fail(CA_ERR_UNSUPPORTED, "%s: window row bytes not a multiple of 16", what);
  add((uint8_t*)st->window + seq * wrow, nullptr, 0, wrow, 1);
  for (int j = 0; j < st->n_jobs; ++j) {
    if (st->tail[j] == nullptr || st->tail_floats[j] <= 0 || (st->tail_floats[j] * 4) % 16)
      return fail(CA_ERR_ARG, "%s: job %d: bad tail ring", what, j);
    add((uint8_t*)(st->tail[j] + seq * st->tail_floats[j]), nullptr, 0, st->tail_floats[j] * 4, 1);
  }
  for (int j = 0; j < st->n_jobs; ++j) {
    ca::CacheView cv;
    if (int e = make_view(st->cache[j], &cv, what)) return e;
    if (st->ratio[j] <= 0) return fail(CA_ERR_ARG, "%s: job %d: ratio must be positive", what, j);
    if (seq >= st->cache[j]->n_seqs) return fail(CA_ERR_ARG, "%s: job %d: seq beyond the page table", what, j);
    const int64_t n_e = pos / st->ratio[j];
    const int64_t n_pg = (n_e + st->cache[j]->page_size - 1) / st->cache[j]->page_size;
    if (n_pg > st->cache[j]->max_pages) return fail(CA_ERR_ARG, "%s: job %d: %lld pages beyond the page table", what, j,
                                                    (long long)n_pg);
    if (cv.page_bytes % 16 || (uintptr_t)cv.pool % 16)
      return fail(CA_ERR_UNSUPPORTED, "%s: job %d: pool or page bytes not 16-byte aligned", what, j);
    add(cv.pool, cv.page_table + (int64_t)seq * cv.max_pages, cv.n_pages, cv.page_bytes, n_pg);
  }
  if (plan) *plan = p;
  *total = off;
  return CA_OK;
}

int64_t ca_state_bytes(const ca_decode_state* st, int64_t pos) {
  int64_t total = 0;
  if (state_plan(st, 0, pos, nullptr, nullptr, &total, "ca_state_bytes")) return -1;
  ok();
  return total;
}

static int state_copy(const ca_decode_state* st, int32_t seq, int64_t pos, void* buffer, int64_t bytes, int to_buffer,
                      void* stream, const char* what) {
  ca::StatePlan p;
  int64_t total = 0;
  if (int e = state_plan(st, seq, pos, buffer, &p, &total, what)) return e;
  if (buffer == nullptr || bytes < total)
    return fail(CA_ERR_WORKSPACE, "%s: buffer of %lld bytes < %lld needed", what, (long long)bytes, (long long)total);
  return hip_status(ca::launch_state_copy(p, to_buffer, S(stream)), what);
}

int ca_state_save(const ca_decode_state* st, int32_t seq, int64_t pos, void* buffer, int64_t buffer_bytes,
                  void* stream) {
  return state_copy(st, seq, pos, buffer, buffer_bytes, 1, stream, "ca_state_save");
}

int ca_state_load(const ca_decode_state* st, int32_t seq, int64_t pos, const void* buffer, int64_t buffer_bytes,
                  void* stream) {
  return state_copy(st, seq, pos, (void*)buffer, buffer_bytes, 0, stream, "ca_state_load");
}

int ca_attend_decode_plan(const ca_attend_params* p, int64_t total, int32_t* chunk_len, int32_t* n_chunks,
                          int32_t* max_chunks) {
  if (p == nullptr || total < 0 || total > 0x7FFFFFFF || chunk_len == nullptr || n_chunks == nullptr)
    return fail(CA_ERR_ARG, "ca_attend_decode_plan: bad arguments");
  const int cap = ca::attend_mfma_max_items();
  int mn, dv;
  decode_plan_of(p->n_heads, p->dim, p->rope_dim, &mn, &dv);
  *chunk_len = ca::split_plan_len(total, mn, dv, cap);
  *n_chunks = ca::split_plan_count(total, mn, dv, cap);
  if (max_chunks) *max_chunks = ca::plan_max_splits(total, mn, dv, cap);
  return ok();
}

static int attend_common(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                         int mode, int seq_fixed, const int32_t* pos, int64_t t0, int64_t n_rows, int64_t max_pos,
                         const int32_t* idx, const int32_t* cnt, int k, int ratio, const void* window, int W,
                         int win_rows, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream, bool decode, const char* what, ca::AttendArgs* plan = nullptr) {
  if (plan) plan->n_rows = 0;
  if (p == nullptr) return fail(CA_ERR_ARG, "%s: params NULL", what);
  ca::AttendArgs a;
  if (int e = make_view(kv, &a.kv, what)) return e;
  if (kv->format != CA_F32 && kv->format != CA_BF16 && kv->format != CA_FP8MIX)
    return fail(CA_ERR_DTYPE, "%s: main KV pool must be F32, BF16 or FP8MIX", what);
  if (p->dim != kv->dim || p->rope_dim != kv->rope_dim)
    return fail(CA_ERR_ARG, "%s: params dim/rope_dim differ from the cache", what);
  if (p->dim % 64 != 0 || (p->dim / 64 != 1 && p->dim / 64 != 2 && p->dim / 64 != 4 && p->dim / 64 != 8))
    return fail(CA_ERR_UNSUPPORTED, "%s: dim must be 64, 128, 256 or 512", what);
  if (p->n_heads <= 0 || p->n_win < 1) return fail(CA_ERR_ARG, "%s: n_heads and n_win must be positive", what);
  if (!is_act(p->q_format) || !is_act(p->win_format) || !is_act(p->out_format))
    return fail(CA_ERR_DTYPE, "%s: q/window/out formats must be F32 or BF16", what);
  if (ratio <= 0) return fail(CA_ERR_ARG, "%s: ratio must be positive", what);
  if (mode == 0 && k <= 0) return fail(CA_ERR_ARG, "%s: k must be positive", what);
  if (n_rows < 0 || n_rows > 0x7FFFFFFF || W <= 0) return fail(CA_ERR_ARG, "%s: bad sizes", what);
  if (n_rows == 0) return ok();
  if (!q || !q_gain || !window || !sink || !out) return fail(CA_ERR_ARG, "%s: NULL argument", what);
  if (mode == 0 && (!idx || !cnt)) return fail(CA_ERR_ARG, "%s: idx/cnt NULL", what);
  if (decode && !pos) return fail(CA_ERR_ARG, "%s: pos NULL", what);
  if (!decode && (t0 < 0 || t0 + n_rows > 0x7FFFFFFF)) return fail(CA_ERR_ARG, "%s: bad L / t0", what);
  if (!decode && W < n_rows + (t0 < p->n_win - 1 ? t0 : p->n_win - 1))
    return fail(CA_ERR_ARG, "%s: prefill window needs W >= L + min(t0, n_win - 1)", what);
  if (decode && n_rows > kv->n_seqs) return fail(CA_ERR_ARG, "%s: more rows than page table rows", what);
  if (decode && W < p->n_win) return fail(CA_ERR_ARG, "%s: window ring W = %d < n_win = %d", what, W, p->n_win);
  if (max_pos > 0x7FFFFFFF) return fail(CA_ERR_ARG, "%s: max_pos beyond 2^31 - 1", what);
  // the kernels take a row's split plan in 32-bit arithmetic
  if (max_items_of(max_pos, p->n_win, mode == 0 ? k : 0, ratio) > 0x7FFFFFFF - 4096)
    return fail(CA_ERR_UNSUPPORTED, "%s: a row may hold 2^31 - 4096 or more items", what);
  if (mode == 1 && max_pos / ratio > (int64_t)kv->max_pages * kv->page_size)
    return fail(CA_ERR_ARG, "%s: page table holds fewer than floor(max_pos/ratio) entries", what);
  // the attention kernels address an item by pool record index (page * page_size + slot) or
  // by window row, in 31 bits: every record and every window row must have an index below
  // 2^31 - 1 (e.g. 1.37 TB of fp8 records)
  if ((int64_t)kv->n_pages * kv->page_size >= 0x7FFFFFFF)
    return fail(CA_ERR_UNSUPPORTED, "%s: pool holds 2^31 - 1 or more records", what);
  if ((int64_t)(decode ? n_rows : 1) * W >= 0x7FFFFFFF)
    return fail(CA_ERR_UNSUPPORTED, "%s: window holds 2^31 - 1 or more rows", what);
  (void)win_rows;
  a.q = q;
  a.q_gain = q_gain;
  a.q_fmt = p->q_format;
  a.n_heads = p->n_heads;
  a.D = p->dim;
  a.R = p->rope_dim;
  a.n_win = p->n_win;
  a.scale_log2 = p->scale * ca::kLog2e;
  a.eps = p->eps;
  a.base = p->rope_base;
  a.rope_step = p->rope_dim > 0 ? pow(p->rope_base, -2.0 / (double)p->rope_dim) : 1.0;
  a.pos = pos;
  a.t0 = (int)t0;
  a.seq_fixed = seq_fixed;
  a.n_rows = (int)n_rows;
  a.mode = mode;
  a.ratio = ratio;
  a.idx = idx;
  a.cnt = cnt;
  a.k = k;
  a.win = window;
  a.win_fmt = p->win_format;
  a.W = W;
  a.sink = sink;
  a.out = out;
  a.out_fmt = p->out_format;
  a.lse = lse;
  a.max_pos = (int)max_pos;
  a.status = p->status;
  a.split_min = 0;
  a.split_div = 1;
  a.split_cap = ca::attend_mfma_max_items();
  a.max_splits = 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.q_prep = nullptr;
  a.q_inv = nullptr;
  // Split the item list of each row into chunks by a plan that depends on the row
  // alone (ca::split_plan_len): always for decode, and for prefill when a row can be
  // longer than one MFMA workgroup's item table.
  const int64_t max_items = max_items_of(max_pos, p->n_win, mode == 0 ? k : 0, ratio);
  int split = 0, div = 1, ms = 1;
  if (decode) {
    decode_plan_of(p->n_heads, p->dim, p->rope_dim, &split, &div);
  } else if (ca::attend_mfma_supported(a) && max_items > ca::attend_mfma_max_items()) {
    split = 64;
    div = 1;
  }
  if (split > 0) ms = ca::plan_max_splits(max_items, split, div, a.split_cap);
  if (split > 0) {
    const size_t po = align256((size_t)n_rows * ms * p->n_heads * p->dim * (p->out_format == CA_BF16 ? 2 : 4));
    const size_t pm = align256((size_t)n_rows * ms * p->n_heads * 2 * sizeof(float));
    const size_t pq = align256((size_t)n_rows * p->n_heads * p->dim * 2);
    const size_t pi = align256((size_t)n_rows * p->n_heads * sizeof(float));
    const size_t need = po + pm + pq + pi;
    if (ws_bytes < need || ws == nullptr)
      return fail(CA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes (rows of up to %lld items are split)", what,
                  ws_bytes, need, (long long)max_items);
    a.split_min = split;
    a.split_div = div;
    a.max_splits = ms;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + po);
    if (ca::attend_mfma_supported(a)) {
      a.q_prep = (uint16_t*)((char*)ws + po + pm);
      a.q_inv = (float*)((char*)ws + po + pm + pq);
    }
  }
  if (plan) {
    *plan = a;
    return CA_OK;
  }
  return hip_status(ca::launch_attend(a, S(stream)), what);
}

int ca_csa_attend_prefill(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                          int32_t seq, const int32_t* idx, const int32_t* cnt, int32_t k, int32_t ratio,
                          const void* window, int32_t W, const float* sink, int64_t L, int64_t t0, void* out,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (kv && (seq < 0 || seq >= kv->n_seqs)) return fail(CA_ERR_ARG, "ca_csa_attend_prefill: seq out of range");
  return attend_common(p, q, q_gain, kv, 0, seq, nullptr, t0, L, t0 + L - 1, idx, cnt, k, ratio, window, W, 1, sink, out, lse,
                       ws, ws_bytes, stream, false, "ca_csa_attend_prefill");
}

int ca_csa_attend_decode(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                         const int32_t* idx, const int32_t* cnt, int32_t k, int32_t ratio, const int32_t* pos,
                         int32_t B, int64_t max_pos, const void* window, int32_t W, const float* sink, void* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attend_common(p, q, q_gain, kv, 0, -1, pos, 0, B, max_pos, idx, cnt, k, ratio, window, W, B, sink, out, lse, ws,
                       ws_bytes, stream, true, "ca_csa_attend_decode");
}

int ca_hca_attend_prefill(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                          int32_t seq, int32_t ratio, const void* window, int32_t W, const float* sink, int64_t L,
                          int64_t t0, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (kv && (seq < 0 || seq >= kv->n_seqs)) return fail(CA_ERR_ARG, "ca_hca_attend_prefill: seq out of range");
  return attend_common(p, q, q_gain, kv, 1, seq, nullptr, t0, L, t0 + L - 1, nullptr, nullptr, 0, ratio, window, W, 1, sink,
                       out, lse, ws, ws_bytes, stream, false, "ca_hca_attend_prefill");
}

int ca_hca_attend_decode(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                         int32_t ratio, const int32_t* pos, int32_t B, int64_t max_pos, const void* window,
                         int32_t W, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  return attend_common(p, q, q_gain, kv, 1, -1, pos, 0, B, max_pos, nullptr, nullptr, 0, ratio, window, W, B, sink, out,
                       lse, ws, ws_bytes, stream, true, "ca_hca_attend_decode");
}

// ------------------------------------------------------------------ decode steps
// A layer's whole decode step: append (+ CSA indexer and top-k) + attention, with
// the query preparation and the top-k state clearing done by the append launch.
static int decode_step(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window, int32_t W,
                       int32_t S_, const ca_decode_entry_job* jobs, int32_t n_jobs, const ca_index_params* ip,
                       const void* qI, const float* wI, int32_t* idx, int32_t* cnt, void* iws, size_t iws_bytes,
                       const ca_attend_params* ap, const void* q, const float* q_gain, const int32_t* pos, int32_t B,
                       int64_t max_pos, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream, bool csa, const char* what) {
  ca::DecodeWindowJob wj;
  ca::DecodeEntryJob ej[2];
  if (int e = append_plan(wp, kv_raw, w_gain, pos, B, window, W, S_, jobs, n_jobs, &wj, ej, what)) return e;
  if (max_pos < 0) return fail(CA_ERR_ARG, "%s: negative max_pos", what);
  IndexPlan iplan;
  iplan.n_rows = 0;
  if (csa) {
    if (ip == nullptr) return fail(CA_ERR_ARG, "%s: index params NULL", what);
    if (ip->ratio != jobs[0].params.ratio || ip->ratio != jobs[1].params.ratio)
      return fail(CA_ERR_ARG, "%s: indexer and compressor ratios differ", what);
    if (int e = index_common(ip, qI, wI, pos, 0, -1, B, max_pos, jobs[1].cache, idx, cnt, nullptr, nullptr, 0, iws,
                             iws_bytes, stream, what, &iplan))
      return e;
  }
  ca::AttendArgs aplan;
  if (int e = attend_common(ap, q, q_gain, jobs[0].cache, csa ? 0 : 1, -1, pos, 0, B, max_pos, idx, cnt,
                            csa ? ip->k : 0, jobs[0].params.ratio, window, W, B, sink, out, lse, ws, ws_bytes, stream,
                            true, what, &aplan))
    return e;
  if (B == 0) return ok();
  uint32_t* zero = iplan.n_rows > 0 && iplan.ws_long != nullptr ? (uint32_t*)iplan.ws_long : nullptr;
  hipError_t e = ca::launch_decode_front(wj, ej, n_jobs, pos, B, aplan.q_prep ? &aplan : nullptr, zero,
                                         zero ? ca::kTopkRowWords : 0, S(stream));
  if (e == hipSuccess && csa) e = launch_index_plan(iplan, S(stream), zero != nullptr);
  if (e == hipSuccess) e = ca::launch_attend(aplan, S(stream), aplan.q_prep != nullptr);
  return hip_status(e, what);
}

int ca_csa_decode_step(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window, int32_t W,
                       int32_t S_, const ca_decode_entry_job* jobs, const ca_index_params* ip, const void* qI,
                       const float* wI, int32_t* idx, int32_t* cnt, void* iws, size_t iws_bytes,
                       const ca_attend_params* ap, const void* q, const float* q_gain, const int32_t* pos, int32_t B,
                       int64_t max_pos, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  return decode_step(wp, kv_raw, w_gain, window, W, S_, jobs, 2, ip, qI, wI, idx, cnt, iws, iws_bytes, ap, q, q_gain,
                     pos, B, max_pos, sink, out, lse, ws, ws_bytes, stream, true, "ca_csa_decode_step");
}

int ca_hca_decode_step(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window, int32_t W,
                       int32_t S_, const ca_decode_entry_job* job, const ca_attend_params* ap, const void* q,
                       const float* q_gain, const int32_t* pos, int32_t B, int64_t max_pos, const float* sink,
                       void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_step(wp, kv_raw, w_gain, window, W, S_, job, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     0, ap, q, q_gain, pos, B, max_pos, sink, out, lse, ws, ws_bytes, stream, false,
                     "ca_hca_decode_step");
}

}  // extern "C"

// ------------------------------------------------------------------ static scratch
// Device scratch of the allocation-free HCA decode step: a file-scope array that
// every device the library runs on holds until the process ends.  In host code its
// name is only a stand-in; its device address is looked up once per device (with
// that device current) and only that address is ever passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on first use).
int scratch_of_current_device(void** out, const char* what) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CA_ERR_HIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CA_ERR_UNSUPPORTED, "%s: device %d beyond %d", what, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", what, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CA_OK;
}
}  // namespace

extern "C" {

size_t ca_static_scratch_bytes(void) { return kStaticScratchBytes; }

int ca_hca_decode_step_noalloc(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window,
                               int32_t W, int32_t S_, const ca_decode_entry_job* job, const ca_attend_params* ap,
                               const void* q, const float* q_gain, const int32_t* pos, int32_t B, int64_t max_pos,
                               const float* sink, void* out, float* lse, void* stream) {
  const char* what = "ca_hca_decode_step_noalloc";
  if (job == nullptr || ap == nullptr) return fail(CA_ERR_ARG, "%s: job or attention params NULL", what);
  if (B < 0 || max_pos < 0) return fail(CA_ERR_ARG, "%s: negative B or max_pos", what);
  const size_t need = B > 0 ? ca_attend_workspace(ap, B, max_pos, 0, job->params.ratio) : 0;
  if (need > kStaticScratchBytes)
    return fail(CA_ERR_WORKSPACE, "%s: the step needs %zu bytes of scratch, the static scratch holds %zu", what, need,
                kStaticScratchBytes);
  if (B == 0) return decode_step(wp, kv_raw, w_gain, window, W, S_, job, 1, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, nullptr, 0, ap, q, q_gain, pos, B, max_pos, sink, out, lse, nullptr, 0,
                                 stream, false, what);
  void* ws = nullptr;
  if (int e = scratch_of_current_device(&ws, what)) return e;
  return decode_step(wp, kv_raw, w_gain, window, W, S_, job, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     0, ap, q, q_gain, pos, B, max_pos, sink, out, lse, ws, kStaticScratchBytes, stream, false, what);
}

}  // extern "C"

// --------------------------------------------------------------- sublayer GEMMs
namespace {

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

ca::GemmSeg gemm_seg(const void* W, void* C, int N, int c_f32, int64_t ldw, int64_t ldc, int64_t w_batch = 0,
                     int64_t c_batch = 0) {
  ca::GemmSeg s{};
  s.W = W;
  s.C = C;
  s.N = N;
  s.c_f32 = c_f32;
  s.ldw = ldw;
  s.ldc = ldc;
  s.w_batch = w_batch;
  s.c_batch = c_batch;
  return s;
}

ca::GemmArgs gemm_args(const void* A, int64_t lda, int M, int K, int batch = 1, int64_t a_batch = 0) {
  ca::GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.a_batch = a_batch;
  g.M = M;
  g.K = K;
  g.batch = batch;
  return g;
}

// The two GEMM stages of the low-rank query projections (pointers may be null when
// only the plan is wanted).
void query_stages(const ca_query_proj_params* p, int M, const void* h, void* c_q, void* q, void* q_i, float* w_i,
                  ca::GemmArgs* g) {
  g[0] = gemm_args(h, p->d, M, p->d);
  g[0].seg[0] = gemm_seg(p->w_dq, c_q, p->d_c, 0, p->d, p->d_c);
  g[0].seg[1] = gemm_seg(p->w_w, w_i, p->n_i, 1, p->d, p->n_i);
  g[0].n_seg = p->n_i > 0 ? 2 : 1;
  g[1] = gemm_args(c_q, p->d_c, M, p->d_c);
  g[1].seg[0] = gemm_seg(p->w_uq, q, p->n_q, 0, p->d_c, p->n_q);
  g[1].seg[1] = gemm_seg(p->w_iuq, q_i, p->n_qi, 0, p->d_c, p->n_qi);
  g[1].n_seg = p->n_qi > 0 ? 2 : 1;
}

void out_stages(const ca_out_proj_params* p, int M, const void* o, void* u, void* y, ca::GemmArgs* g) {
  const int G = p->n_h / 8, width = 8 * p->c;
  g[0] = gemm_args(o, (int64_t)p->n_h * p->c, M, width, G, width);
  g[0].seg[0] = gemm_seg(p->w_o1, u, p->d_g, 0, width, (int64_t)G * p->d_g, (int64_t)p->d_g * width, p->d_g);
  g[0].n_seg = 1;
  g[1] = gemm_args(u, (int64_t)G * p->d_g, M, G * p->d_g);
  g[1].seg[0] = gemm_seg(p->w_o2, y, p->d, 0, (int64_t)G * p->d_g, p->d);
  g[1].n_seg = 1;
}

size_t stages_workspace(ca::GemmArgs* g, int n) {
  int64_t f = 0;
  for (int i = 0; i < n; ++i) {
    ca::gemm_plan(g[i]);
    f = g[i].part_floats > f ? g[i].part_floats : f;
  }
  return (size_t)f * sizeof(float);
}

int check_query(const ca_query_proj_params* p, int64_t T, const char* what) {
  if (p == nullptr) return fail(CA_ERR_ARG, "%s: params NULL", what);
  if (T < 0 || T > INT32_MAX) return fail(CA_ERR_ARG, "%s: T outside 0..2^31-1", what);
  if (p->d <= 0 || p->d_c <= 0 || p->n_q <= 0 || p->n_qi < 0 || p->n_i < 0 || (p->n_qi > 0) != (p->n_i > 0))
    return fail(CA_ERR_ARG, "%s: bad widths (n_qi and n_i are both 0 or both positive)", what);
  if (p->d % 64 || p->d_c % 64) return fail(CA_ERR_UNSUPPORTED, "%s: d and d_c must be multiples of 64", what);
  if (!p->w_dq || !p->w_uq || (p->n_qi > 0 && (!p->w_iuq || !p->w_w)))
    return fail(CA_ERR_ARG, "%s: NULL weight", what);
  if (!al16(p->w_dq) || !al16(p->w_uq) || (p->n_qi > 0 && (!al16(p->w_iuq) || !al16(p->w_w))))
    return fail(CA_ERR_ARG, "%s: weights must be 16-byte aligned", what);
  return 0;
}

int check_out(const ca_out_proj_params* p, int64_t T, const char* what) {
  if (p == nullptr) return fail(CA_ERR_ARG, "%s: params NULL", what);
  if (T < 0 || T > INT32_MAX) return fail(CA_ERR_ARG, "%s: T outside 0..2^31-1", what);
  if (p->n_h <= 0 || p->c <= 0 || p->d_g <= 0 || p->d <= 0) return fail(CA_ERR_ARG, "%s: bad widths", what);
  if (p->n_h % 8) return fail(CA_ERR_UNSUPPORTED, "%s: n_h must be a multiple of 8 (8 heads a group)", what);
  if ((8 * p->c) % 64 || ((p->n_h / 8) * p->d_g) % 64)
    return fail(CA_ERR_UNSUPPORTED, "%s: 8 c and g d_g must be multiples of 64", what);
  if (!p->w_o1 || !p->w_o2) return fail(CA_ERR_ARG, "%s: NULL weight", what);
  if (!al16(p->w_o1) || !al16(p->w_o2)) return fail(CA_ERR_ARG, "%s: weights must be 16-byte aligned", what);
  return 0;
}

int run_stages(ca::GemmArgs* g, int n, void* ws, size_t ws_bytes, void* stream, const char* what) {
  const size_t need = stages_workspace(g, n);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(CA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", what, ws_bytes, need);
  for (int i = 0; i < n; ++i) {
    g[i].part = (float*)ws;
    if (int e = hip_status(ca::launch_gemm(g[i], S(stream)), what)) return e;
  }
  return ok();
}

}  // namespace

extern "C" {

size_t ca_query_proj_workspace(const ca_query_proj_params* p, int64_t T) {
  if (check_query(p, T, "ca_query_proj_workspace")) return 0;
  ca::GemmArgs g[2];
  query_stages(p, (int)T, nullptr, nullptr, nullptr, nullptr, nullptr, g);
  return stages_workspace(g, 2);
}

int ca_query_proj(const ca_query_proj_params* p, const void* h, int64_t T, void* c_q, void* q, void* q_i, float* w_i,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "ca_query_proj";
  if (int e = check_query(p, T, what)) return e;
  if (T == 0) return ok();
  if (!h || !c_q || !q || (p->n_qi > 0 && (!q_i || !w_i))) return fail(CA_ERR_ARG, "%s: NULL buffer", what);
  if (!al16(h) || !al16(c_q)) return fail(CA_ERR_ARG, "%s: h and c_q must be 16-byte aligned", what);
  ca::GemmArgs g[2];
  query_stages(p, (int)T, h, c_q, q, q_i, w_i, g);
  return run_stages(g, 2, workspace, workspace_bytes, stream, what);
}

size_t ca_out_proj_workspace(const ca_out_proj_params* p, int64_t T) {
  if (check_out(p, T, "ca_out_proj_workspace")) return 0;
  ca::GemmArgs g[2];
  out_stages(p, (int)T, nullptr, nullptr, nullptr, g);
  return stages_workspace(g, 2);
}

int ca_out_proj(const ca_out_proj_params* p, const void* o, int64_t T, void* u, void* y, void* workspace,
                size_t workspace_bytes, void* stream) {
  const char* what = "ca_out_proj";
  if (int e = check_out(p, T, what)) return e;
  if (T == 0) return ok();
  if (!o || !u || !y) return fail(CA_ERR_ARG, "%s: NULL buffer", what);
  if (!al16(o) || !al16(u)) return fail(CA_ERR_ARG, "%s: o and u must be 16-byte aligned", what);
  ca::GemmArgs g[2];
  out_stages(p, (int)T, o, u, y, g);
  return run_stages(g, 2, workspace, workspace_bytes, stream, what);
}

}  // extern "C"
