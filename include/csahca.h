/*
 * csahca.h -- C ABI of the MI355X (gfx950) library for compressed sparse
 * attention (CSA) and heavily compressed attention (HCA), prefill and decode,
 * over a paged compressed-KV cache.
 *
 * The method is the one described in the DeepSeek-V4 technical-report
 * walkthrough book (slop-6tp.pages.dev/papers-html-argon/dsv4.html, "dsv4
 * book" below), chapters 5-8.  Each entry point cites the passage that defines
 * the operation it runs.
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers owned by the caller unless a comment says
 *    "host".  The library never allocates memory: scratch space is passed in
 *    (`ws`, `ws_bytes`) after asking the matching *_workspace function.
 *  - `stream` is a hipStream_t passed as void*; every call only enqueues work
 *    on it (no host synchronisation), so calls can be captured in HIP graphs.
 *  - Every call returns a ca_status.  Arguments are validated on the host
 *    before anything is launched; on error nothing is launched and
 *    ca_last_error() (thread-local) describes the problem.
 *  - Row-major layouts throughout.  "bf16" is bfloat16, "e4m3" is OCP FP8
 *    E4M3 (fn variant: no infinities, max 448).
 *  - Results are bitwise deterministic and, for decode, independent of which
 *    other sequences share the batch and of the host max_pos bound.
 */
#ifndef CSAHCA_H
#define CSAHCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_ERR_ARG = -1,          /* null pointer, negative size, inconsistent shape */
  CA_ERR_DTYPE = -2,        /* unsupported storage format for this argument */
  CA_ERR_UNSUPPORTED = -3,  /* valid but not implemented (e.g. dim not a multiple of 64) */
  CA_ERR_WORKSPACE = -4,    /* workspace too small */
  CA_ERR_HIP = -5           /* a HIP launch failed */
} ca_status;

/* Device status bits.  Calls whose params carry a `status` pointer (a device
 * int32 owned by the caller) OR these bits into it from the kernels, for
 * conditions the host cannot see because they depend on device data.  The
 * library never clears the word; nothing is reported when `status` is NULL.
 *   CA_STATUS_POS_RANGE: a decode row's position pos[b] is negative or larger
 *     than the call's max_pos.  The row is out of contract and treated as
 *     empty: the indexer keeps no entry for it (cnt 0, idx all -1) and the
 *     attention writes a zero output row (lse = the sink logit); nothing
 *     outside the caller's buffers is read or written. */
enum { CA_STATUS_POS_RANGE = 1 };

/* Storage formats. */
typedef enum {
  CA_F32 = 0,     /* float32 */
  CA_BF16 = 1,    /* bfloat16 */
  CA_FP8MIX = 2,  /* main-KV record: e4m3 content channels + bf16 rotary channels (see ca_cache) */
  CA_E4M3 = 3,    /* indexer-key page: e4m3 codes + one fp32 power-of-two scale per entry */
  CA_FP4 = 4      /* indexer-key page: e2m1 codes + one E8M0 scale per 32 channels */
} ca_format;

/* Thread-local description of the last error (empty string if none). */
const char* ca_last_error(void);

/* ------------------------------------------------------------------------ */
/* Paged compressed cache (dsv4 book Ch.5 "Decode-time cache state"; Ch.8    */
/* "V4 compressed-entry payload" and "Quantization scales and bounded tail   */
/* buffers").  Completed entries are append-only; entry i of sequence s lives */
/* in page page_table[s * max_pages + i / page_size], slot i % page_size.     */
/*                                                                           */
/* Record formats (one entry = one record; a page is page_size records):     */
/*   CA_F32    : dim float32 (stride 4*dim bytes)                            */
/*   CA_BF16   : dim bf16   (stride 2*dim bytes)                             */
/*   CA_FP8MIX : bytes [0, dim-R)          e4m3 codes of content channels     */
/*               bytes [dim-R, dim+R)      bf16 rotary channels (R = rope_dim)*/
/*               bytes [dim+R, +(dim-R)/64) int8 exponent e of each 64-channel*/
/*                                         content tile (value = code * 2^e)  */
/*               zero padding up to a multiple of 128 bytes (640 for 512/64). */
/*   CA_E4M3   : indexer pages, structure of arrays: page_size*dim codes,     */
/*               then page_size float32 scales (powers of two).              */
/*   CA_FP4    : indexer pages (Ch.8: FP4 keys, a 1-byte scale per 32        */
/*               elements), structure of arrays: page_size*dim/2 bytes of    */
/*               OCP e2m1 codes (channel 2c in the low nibble of byte c),    */
/*               then page_size*dim/32 E8M0 bytes (block b of slot i at      */
/*               i*dim/32 + b; value 2^(byte-127)).  Element = code * scale, */
/*               the scale the smallest power of two with block max <= 6 *   */
/*               scale; codes rounded to nearest, ties to even.  dim % 32 == 0*/
/* A page table entry < 0 or >= n_pages marks a missing page: entries in it  */
/* are never read (kernels skip them) and never written.                     */
/* ------------------------------------------------------------------------ */
typedef struct ca_cache {
  int32_t format;             /* ca_format of the records in `pool` */
  int32_t dim;                /* D (main KV) or c_I (indexer keys) */
  int32_t rope_dim;           /* R, the rotary channels at the end of each main entry; 0 for indexer pools */
  int32_t page_size;          /* entries per page (64 in the presets) */
  void* pool;                 /* device, n_pages * ca_page_bytes(format, dim, rope_dim, page_size) bytes */
  int64_t n_pages;
  const int32_t* page_table;  /* device, [n_seqs, max_pages] int32 */
  int32_t n_seqs;
  int32_t max_pages;
} ca_cache;

/* Bytes of one record / one page of a pool (host helpers, no device work).
 * Return -1 for an unsupported combination. */
int64_t ca_record_stride(int32_t format, int32_t dim, int32_t rope_dim);
int64_t ca_page_bytes(int32_t format, int32_t dim, int32_t rope_dim, int32_t page_size);

/* ------------------------------------------------------------------------ */
/* Entry epilogue + store (dsv4 book Ch.7 "Query and KV RMSNorm", "Partial   */
/* RoPE and output de-rotation"; Ch.8 "V4 compressed-entry payload").        */
/* For k in [0, n): x = src[k] (float32 [n, dim]); optionally               */
/* x <- x / sqrt(mean(x^2) + eps) * gain; optionally rotate the last        */
/* rope_dim channels pairwise (2p, 2p+1) by angle (pos_stride*i)*base^(-2p/R)*/
/* with i = first + k; then encode into entry i of sequence `seq`.          */
/* gain == NULL skips the norm.  Used to build caches directly from vectors. */
/* ------------------------------------------------------------------------ */
int ca_store_entries(const ca_cache* cache, int32_t seq, int64_t first, int64_t n, const float* src,
                     const float* gain, float eps, int32_t apply_rope, double rope_base, int32_t pos_stride,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Sequence compressor (dsv4 book Ch.5 "The four compression projections",  */
/* "Coordinate-wise softmax pooling", "Receptive field versus compression   */
/* stride"; Ch.7 "HCA's 128:1 non-overlapping compressor").                 */
/* overlap = 1 (CSA): entry i, channel r = softmax over the 2m logits        */
/*   Za[m*i+j, r] + Ba[j, r] and Zb[m*(i-1)+j, r] + Bb[j, r] (j < m) of the  */
/*   matching Ca / Cb contents; for i = 0 the b-branch is absent.            */
/* overlap = 0 (HCA): softmax over the m rows Za[m*i+j, r] + Ba[j, r] of Ca. */
/* Only completed blocks are emitted.  The epilogue (RMSNorm with `gain`,    */
/* RoPE at position ratio*i) follows when enabled, then the record encode.   */
/* ------------------------------------------------------------------------ */
typedef struct ca_compress_params {
  int32_t ratio;       /* m (CSA) or m' (HCA) */
  int32_t overlap;     /* 1: CSA overlapping 2m window, 0: disjoint blocks */
  int32_t in_format;   /* CA_F32 or CA_BF16: storage of the projection rows */
  int32_t apply_norm;  /* 1: RMSNorm with gain (main KV); 0: none (indexer keys) */
  int32_t apply_rope;  /* 1: RoPE of the last rope_dim channels at position ratio*i */
  float eps;
  double rope_base;
} ca_compress_params;

/* Prefill: rows [L, cache->dim] of Ca, Za (and Cb, Zb when overlap) in
 * in_format hold positions t0 .. t0+L-1 of sequence `seq`; Ba, Bb float32
 * [ratio, dim].  Writes every entry completed by position t0+L-1 whose pooling
 * window lies inside the rows: entries 0..floor(L/ratio)-1 for t0 = 0; for
 * t0 > 0 (a prefill that continues a reused prefix, infra transcript: the
 * compressed entries are reloaded and the tokens of the incomplete tail block
 * recomputed) entries from ceil(t0/ratio) (+1 when overlapping: entry i also
 * reads the block before it) on.  So to extend a cache holding entries
 * < E, pass rows from t0 = ratio*E (HCA) or ratio*(E-1) (CSA, E >= 1).
 * Cb, Zb, Bb may be NULL when overlap == 0. */
int ca_compress_prefill(const ca_compress_params* p, const void* Ca, const void* Za, const void* Cb,
                        const void* Zb, const float* Ba, const float* Bb, const float* gain, int64_t L, int64_t t0,
                        int32_t seq, const ca_cache* cache, void* stream);

/* Decode (dsv4 book Ch.5 "Decode-time cache state": bounded tail buffers).
 * For each sequence b: the new token at position pos[b] brings rows
 * new_rows[b] ([narr, dim], in_format; narr = 4 for CSA in the order
 * Ca, Cb, Za, Zb, and 2 for HCA in the order C, Z).  They are written to the
 * float32 tail ring tail[b, pos[b] % span, :, :] ([B, span, narr, dim], span =
 * 2m for CSA, m for HCA).  When (pos[b] + 1) % ratio == 0 the completed entry
 * i = (pos[b] + 1) / ratio - 1 is pooled from the ring and stored in sequence
 * b of the cache (usable from position pos[b] + 1 on). */
int ca_compress_decode(const ca_compress_params* p, const void* new_rows, const int32_t* pos, int32_t B,
                       float* tail, const float* Ba, const float* Bb, const float* gain, const ca_cache* cache,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* Sliding window (dsv4 book Ch.7 "The 128-token uncompressed sliding       */
/* window"): each raw token KV row is RMSNorm-ed with `gain`, its last      */
/* rope_dim channels rotated at the token's own position, and stored at     */
/* window[seq, pos % W, :] (window is [S, W, dim] in win_format).  Prefill  */
/* uses W >= L (one slot per position); decode a ring of W >= n_win slots. */
/* ------------------------------------------------------------------------ */
typedef struct ca_window_params {
  int32_t dim;
  int32_t rope_dim;
  int32_t in_format;   /* CA_F32 or CA_BF16 raw rows */
  int32_t win_format;  /* CA_F32 or CA_BF16 window storage */
  float eps;
  double rope_base;
} ca_window_params;

/* kv_raw [T, dim]; pos [T] int32 (NULL: pos = row index); seq [T] int32
 * (NULL: every row is sequence 0). */
int ca_window_append(const ca_window_params* p, const void* kv_raw, const float* gain, const int32_t* pos,
                     const int32_t* seq, int32_t T, void* window, int32_t W, int32_t S, void* stream);

/* ------------------------------------------------------------------------ */
/* Fused decode append: one decode step's token-level cache updates of one  */
/* layer in a single launch (Ch.5 "Decode-time cache state": the window and */
/* the bounded tail buffers).  For every row b (sequence b, position        */
/* pos[b]) it does exactly what these calls do, bit for bit:                */
/*   ca_window_append(wp, kv_raw, w_gain, pos, seq = {0, 1, .., B-1}, B,     */
/*                    window, W, S, stream), and for each of the n_jobs      */
/*   (1 or 2) jobs ca_compress_decode(&job.params, job.new_rows, pos, B,     */
/*                    job.tail, job.Ba, job.Bb, job.gain, job.cache, stream) */
/* (CSA: the main entry and the indexer key; HCA: the entry).  kv_raw:     */
/* [B, wp->dim] raw rows of the new tokens (wp->in_format); window:         */
/* [S, W, wp->dim] ring (wp->win_format); pos: [B] int32.  The jobs must    */
/* not share a tail ring or a cache.  S >= B.  Errors: as the separate      */
/* calls (job index in the message); nothing is launched on an error.       */
/* ------------------------------------------------------------------------ */
typedef struct ca_decode_entry_job {
  ca_compress_params params;
  const void* new_rows;   /* [B, narr, dim] as for ca_compress_decode */
  float* tail;            /* [B, span, narr, dim] float32 tail ring */
  const float* Ba;        /* [ratio, dim] */
  const float* Bb;        /* [ratio, dim] (overlap only, else may be NULL) */
  const float* gain;      /* [dim] (apply_norm only, else may be NULL) */
  const ca_cache* cache;
} ca_decode_entry_job;

int ca_decode_append(const ca_window_params* wp, const void* kv_raw, const float* w_gain, const int32_t* pos,
                     int32_t B, void* window, int32_t W, int32_t S, const ca_decode_entry_job* jobs, int32_t n_jobs,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Lightning indexer + top-k (dsv4 book Ch.6 "The lightning indexer",       */
/* "Top-k selection and asymptotic scaling"; Ch.5 "Causal availability").   */
/* For query row r at position t: for every block s < floor(t/m),           */
/*   I[r, s] = sum_h w[r, h] * ReLU(qI[r, h, :] . K[s, :])                   */
/* with K read from the indexer pool.  For CA_E4M3 and CA_FP4 pools the    */
/* query is first quantized to e4m3 with one power-of-two scale per (row,   */
/* head), exactly (FP4 pools: fp8 queries x FP4 keys, Ch.8).  With         */
/* q_quant = CA_FP4 (FP4 pools only) the query is quantized like the keys  */
/* instead: e2m1 codes rounded to nearest (ties to even) with one E8M0     */
/* power of two per 32 channels, the smallest that keeps the block maximum  */
/* within 6 times it (Ch.6 "The lightning indexer": the indexer in FP4).    */
/* The min(k, floor(t/m)) blocks with the largest score are kept (ties: the */
/* lower block index), written ascending to out_idx[r, :], padded with -1;  */
/* out_cnt[r] is their number.  out_score (optional, [rows, k]) receives    */
/* the score of each kept block; all_scores (optional, [rows,               */
/* all_scores_stride]) receives every eligible score.                       */
/* ------------------------------------------------------------------------ */
typedef struct ca_index_params {
  int32_t n_heads;   /* n_I */
  int32_t dim;       /* c_I (must equal idx_cache->dim) */
  int32_t ratio;     /* m */
  int32_t k;         /* top-k */
  int32_t q_format;  /* CA_F32 or CA_BF16 storage of qI */
  int32_t q_quant;   /* 0: e4m3 queries for E4M3 / FP4 pools (none for F32);
                        CA_FP4: FP4 queries (FP4 pools only; else CA_ERR_ARG) */
  int32_t* status;   /* optional device int32 status word (CA_STATUS_* bits), or NULL */
} ca_index_params;

/* Workspace for either indexer call with n_rows query rows whose positions
 * are at most max_pos. */
size_t ca_index_topk_workspace(const ca_index_params* p, int32_t n_rows, int64_t max_pos);

/* Prefill: rows are positions t0..t0+L-1 of sequence `seq` (t0 > 0: the
 * continuation of a prefix whose entries the cache already holds); qI
 * [L, n_I, c_I], w float32 [L, n_I]; workspace sized for max_pos = t0+L-1. */
int ca_index_topk_prefill(const ca_index_params* p, const void* qI, const float* w, int64_t L, int64_t t0,
                          int32_t seq, const ca_cache* idx_cache, int32_t* out_idx, int32_t* out_cnt,
                          float* out_score, float* all_scores, int64_t all_scores_stride, void* ws, size_t ws_bytes,
                          void* stream);

/* Decode: row b is sequence b at position pos[b] (device int32 [B]);
 * max_pos (host) bounds every pos[b] (a row outside [0, max_pos] is kept
 * empty and raises CA_STATUS_POS_RANGE). */
int ca_index_topk_decode(const ca_index_params* p, const void* qI, const float* w, const int32_t* pos,
                         int32_t B, int64_t max_pos, const ca_cache* idx_cache, int32_t* out_idx,
                         int32_t* out_cnt, float* out_score, float* all_scores, int64_t all_scores_stride,
                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Core attention (dsv4 book Ch.6 "Shared key-value MQA"; Ch.7 "Dense       */
/* attention over heavily compressed history", "The 128-token uncompressed  */
/* sliding window", "Query and KV RMSNorm", "Partial RoPE and output        */
/* de-rotation", "Learned attention sinks"; Ch.2 "What an attention head    */
/* computes" for the 1/sqrt(c) logit scale).  For query row r at position t */
/* and head h:                                                              */
/*   q^ = RoPE_t(RMSNorm(q[r, h, :]; q_gain))                                */
/*   X  = {compressed entries} U {window tokens max(0, t-n_win+1) .. t}      */
/*        CSA: entries idx[r, 0..cnt[r]);  HCA: entries 0..floor(t/m')-1     */
/*   o  = sum_x e^{scale q^.x} x / (sum_x e^{scale q^.x} + e^{sink[h]})      */
/*   out[r, h, :] = o with its last rope_dim channels rotated by R_{-t}.     */
/* Every entry is both key and value.  Window tokens are read as stored by  */
/* ca_window_append.  CSA indices outside [0, floor(t/m)) or in missing     */
/* pages are skipped.  lse (optional, float32 [rows, n_heads]) receives     */
/* log(sum_x e^{scale q^.x} + e^{sink}).                                   */
/* Limits: the pool's records (n_pages * page_size) and the window's rows   */
/* (decode: rows * W; prefill: W) must number fewer than 2^31 - 1, else     */
/* CA_ERR_UNSUPPORTED (items are addressed by 31-bit record / row index).  */
/* ------------------------------------------------------------------------ */
typedef struct ca_attend_params {
  int32_t n_heads;
  int32_t dim;         /* D (must equal kv->dim) */
  int32_t rope_dim;    /* R */
  int32_t n_win;
  int32_t q_format;    /* CA_F32 or CA_BF16 */
  int32_t win_format;  /* CA_F32 or CA_BF16 */
  int32_t out_format;  /* CA_F32 or CA_BF16 */
  float scale;         /* logit scale, 1/sqrt(D) */
  float eps;           /* RMSNorm eps of the query */
  double rope_base;
  int32_t* status;     /* optional device int32 status word (CA_STATUS_* bits), or NULL */
} ca_attend_params;

/* Workspace for an attention call over n_rows rows whose positions are at
 * most max_pos; k = top-k for CSA, 0 for HCA; ratio = m or m'. */
size_t ca_attend_workspace(const ca_attend_params* p, int32_t n_rows, int64_t max_pos, int32_t k, int32_t ratio);

/* CSA prefill: rows are positions t0..t0+L-1 of sequence `seq`;
 * q [L, n_heads, D]; idx [L, k], cnt [L]; window [1, W, D] holding position
 * p at slot p % W for every p in [max(0, t0-n_win+1), t0+L), so
 * W >= L + min(t0, n_win-1). */
int ca_csa_attend_prefill(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                          int32_t seq, const int32_t* idx, const int32_t* cnt, int32_t k, int32_t ratio,
                          const void* window, int32_t W, const float* sink, int64_t L, int64_t t0, void* out,
                          float* lse, void* ws, size_t ws_bytes, void* stream);

/* CSA decode: row b is sequence b at position pos[b]; q [B, n_heads, D];
 * idx [B, k], cnt [B]; window ring [B, W, D] with W >= n_win (CA_ERR_ARG
 * otherwise: slots would alias); max_pos (host) bounds pos (a row outside
 * [0, max_pos] gets a zero output and raises CA_STATUS_POS_RANGE).
 * Decode splits each row's items into chunks by a plan that depends on the
 * row's own item count only, so a row's result is bitwise the same whatever
 * other rows share the batch (and whatever max_pos is). */
int ca_csa_attend_decode(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                         const int32_t* idx, const int32_t* cnt, int32_t k, int32_t ratio, const int32_t* pos,
                         int32_t B, int64_t max_pos, const void* window, int32_t W, const float* sink, void* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream);

/* HCA prefill: rows t = t0..t0+L-1 of sequence `seq` attend entries
 * 0..floor(t/ratio)-1 and the window (as for CSA prefill). */
int ca_hca_attend_prefill(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                          int32_t seq, int32_t ratio, const void* window, int32_t W, const float* sink, int64_t L,
                          int64_t t0, void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Host: the split plan decode attention with params p uses for a row of
 * `total` items (its entries plus its window tokens): *chunk_len items per
 * chunk (the last one shorter) and *n_chunks chunks.  A function of `total`
 * alone (up to 16 chunks of at least 256 items; longer rows get more chunks,
 * each at most 2,176 items); each chunk's partial result is merged in chunk
 * order.
 * *max_chunks (optional) receives the most chunks any row of at most `total`
 * items gets (what the workspace holds per row).  CA_ERR_ARG for total < 0
 * or NULL arguments. */
int ca_attend_decode_plan(const ca_attend_params* p, int64_t total, int32_t* chunk_len, int32_t* n_chunks,
                          int32_t* max_chunks);

/* HCA decode: row b is sequence b at position pos[b] (as for CSA decode). */
int ca_hca_attend_decode(const ca_attend_params* p, const void* q, const float* q_gain, const ca_cache* kv,
                         int32_t ratio, const int32_t* pos, int32_t B, int64_t max_pos, const void* window,
                         int32_t W, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------ */
/* Decode state save / restore (dsv4 book Ch.5 "Decode-time cache state";    */
/* infra transcript: the KV cache is split into a classical cache of        */
/* compressed entries and a state cache -- the recent uncompressed window   */
/* and the compressors' unfinished blocks -- and reused prefixes reload     */
/* them).  One layer's decode state of sequence `seq` after it has consumed */
/* `pos` tokens (its next token sits at position pos) is: its window ring   */
/* row window[seq] ([W, win_dim] in win_format), for each of the layer's    */
/* n_jobs compressors its tail ring tail[j][seq] ([span, narr, dim] fp32,   */
/* tail_floats[j] floats) and the pages holding its pos / ratio[j]          */
/* completed entries of cache[j] (whole pages, in page-table order).        */
/* ca_state_save copies them into one flat device buffer; ca_state_load     */
/* copies such a buffer into sequence `seq` of a layer with the same        */
/* shapes, whose page table may name other pages (resume in another slot or */
/* after the pages were given away).  Decode then continues bit for bit as  */
/* it would have without the round trip (the buffer can go through host     */
/* memory or storage in between: it holds no pointers).  Pages missing on   */
/* the side read from or written to are skipped.  Both calls only enqueue   */
/* one copy kernel on `stream`; buffer: ca_state_bytes(...) bytes.          */
/* ------------------------------------------------------------------------ */
typedef struct ca_decode_state {
  void* window;                 /* device [S, W, win_dim] ring of the layer */
  int32_t W, S, win_dim, win_format;
  int32_t n_jobs;               /* 1 (HCA) or 2 (CSA: main entries, indexer keys) */
  float* tail[2];               /* device [S, tail_floats[j]] fp32 tail rings */
  int64_t tail_floats[2];       /* span * narr * dim of each job's ring per sequence */
  const ca_cache* cache[2];     /* the jobs' paged caches */
  int32_t ratio[2];             /* entries completed after pos tokens: pos / ratio[j] */
} ca_decode_state;

/* Bytes of the flat buffer for a sequence that has consumed pos tokens; -1 on
 * invalid arguments (see ca_last_error). */
int64_t ca_state_bytes(const ca_decode_state* st, int64_t pos);
int ca_state_save(const ca_decode_state* st, int32_t seq, int64_t pos, void* buffer, int64_t buffer_bytes,
                  void* stream);
int ca_state_load(const ca_decode_state* st, int32_t seq, int64_t pos, const void* buffer, int64_t buffer_bytes,
                  void* stream);

/* ------------------------------------------------------------------------ */
/* Launch timing (diagnostics, not part of the method).  While a kernel's   */
/* bit is set, every eager launch of it is bracketed by two HIP events       */
/* recorded on the stream it is launched on; launches inside a stream        */
/* capture are not timed.  Not thread-safe: use from one host thread, with   */
/* no other thread launching library work meanwhile.                         */
typedef enum {
  CA_TIMED_CSA_ATTEND = 0,    /* gathered-entry attention kernel of CSA (one launch per attend call) */
  CA_TIMED_HCA_ATTEND = 1,    /* dense compressed-entry attention kernel of HCA */
  CA_TIMED_INDEX_SCORES = 2,  /* indexer scoring kernel of ca_index_topk_* */
  CA_TIMED_PROJ_GEMM = 3,     /* GEMM kernel of ca_query_proj / ca_out_proj (each GEMM stage one launch) */
  CA_TIMED_KERNELS = 4
} ca_timed_kernel;

/* Start timing the kernels whose bits (1 << ca_timed_kernel) are set in
 * kernel_mask, at most max_launches launches each (later ones run untimed).
 * Creates the HIP events (host call; no device memory).  Discards earlier
 * timings.  CA_ERR_ARG for an unknown bit or max_launches outside 1..2^20. */
int ca_timer_start(uint32_t kernel_mask, int64_t max_launches);

/* Host: waits for the kernel's last timed launch, then returns the summed
 * event-to-event time of its timed launches (ms) and their count. */
int ca_timer_read(int32_t kernel, double* total_ms, int64_t* launches);

/* Waits for pending timed launches, destroys the events, stops timing. */
int ca_timer_stop(void);

/* ------------------------------------------------------------------------ */
/* Decode steps: a layer's whole decode step in one call, for callers that  */
/* run the layer as one unit (Ch.5 "Decode-time cache state", Ch.6, Ch.7).  */
/* ca_csa_decode_step does what these calls do, in this order, with the    */
/* same results bit for bit:                                                */
/*   ca_decode_append(wp, kv_raw, w_gain, pos, B, window, W, S, jobs, 2)    */
/*     (jobs[0]: the main entry, jobs[1]: the indexer key);                 */
/*   ca_index_topk_decode(ip, qI, wI, pos, B, max_pos, jobs[1].cache, idx,  */
/*     cnt, NULL, NULL, 0, iws, iws_bytes);                                 */
/*   ca_csa_attend_decode(ap, q, q_gain, jobs[0].cache, idx, cnt, ip->k,    */
/*     jobs[0].params.ratio, pos, B, max_pos, window, W, sink, out, lse,    */
/*     ws, ws_bytes).                                                       */
/* ca_hca_decode_step likewise runs ca_decode_append with its one job and   */
/* ca_hca_attend_decode.  Fewer launches: the append launch also prepares   */
/* the attention queries of split rows and clears the long top-k state.    */
/* Arguments, workspaces and errors: those of the calls above (checked      */
/* before anything is launched); ip->ratio must equal both jobs' ratios.    */
/* ------------------------------------------------------------------------ */
int ca_csa_decode_step(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window, int32_t W,
                       int32_t S, const ca_decode_entry_job* jobs, const ca_index_params* ip, const void* qI,
                       const float* wI, int32_t* idx, int32_t* cnt, void* iws, size_t iws_bytes,
                       const ca_attend_params* ap, const void* q, const float* q_gain, const int32_t* pos, int32_t B,
                       int64_t max_pos, const float* sink, void* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream);
int ca_hca_decode_step(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window, int32_t W,
                       int32_t S, const ca_decode_entry_job* job, const ca_attend_params* ap, const void* q,
                       const float* q_gain, const int32_t* pos, int32_t B, int64_t max_pos, const float* sink,
                       void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Allocation-free HCA decode step, for callers that cannot allocate device  */
/* memory at all (code under HIP graph capture, tight serving loops,         */
/* harnesses that forbid hipMalloc): ca_hca_decode_step with the attention   */
/* workspace taken from a static device array of the library instead of a   */
/* `ws` argument.  Same arguments (minus ws / ws_bytes), results (bit for    */
/* bit) and errors as ca_hca_decode_step; CA_ERR_WORKSPACE when the step     */
/* needs more than ca_static_scratch_bytes() of scratch                      */
/* (ca_attend_workspace(ap, B, max_pos, 0, job->params.ratio) bytes: 64 MiB  */
/* cover e.g. 8 rows x 128 heads at 2^20 tokens or 64 rows x 64 heads at     */
/* 128K tokens).  It calls no allocator.  Each GPU holds one such array      */
/* (from its first call on that device until the process ends) and every    */
/* call on that GPU shares it: calls that overlap on one GPU (concurrent     */
/* streams, threads) race and must be serialized by the caller.  The first  */
/* call on a device looks up the array's device address (host work only).  */
/* ------------------------------------------------------------------------ */
size_t ca_static_scratch_bytes(void);
int ca_hca_decode_step_noalloc(const ca_window_params* wp, const void* kv_raw, const float* w_gain, void* window,
                               int32_t W, int32_t S, const ca_decode_entry_job* job, const ca_attend_params* ap,
                               const void* q, const float* q_gain, const int32_t* pos, int32_t B, int64_t max_pos,
                               const float* sink, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* The attention sublayer around CSA / HCA (dsv4 book Ch.6 "Low-rank query   */
/* generation", "The lightning indexer" and "Grouped output projections";    */
/* Ch.4 "Query head scaling and grouped output projections").  Plain linear  */
/* maps, no bias; bf16 storage, fp32 accumulation.  Weights are [out][in]    */
/* row-major bf16 arrays (the transpose of the pages' x W form), 16-byte     */
/* aligned.  Every width that is summed over (d, d_c, 8 c) must be a         */
/* multiple of 64 (else CA_ERR_UNSUPPORTED); T up to 2^31 - 1 rows.          */
/* ------------------------------------------------------------------------ */
typedef struct ca_query_proj_params {
  int32_t d;          /* hidden width */
  int32_t d_c;        /* query latent width */
  int32_t n_q;        /* main query channels n_h * c */
  int32_t n_qi;       /* indexer query channels n_I * c_I (0: no indexer, HCA) */
  int32_t n_i;        /* indexer heads n_I (combiner weights; 0 with n_qi == 0) */
  const void* w_dq;   /* bf16 [d_c][d]     (W^{DQ}) */
  const void* w_uq;   /* bf16 [n_q][d_c]   (W^{UQ}) */
  const void* w_iuq;  /* bf16 [n_qi][d_c]  (W^{IUQ}) */
  const void* w_w;    /* bf16 [n_i][d]     (W^w) */
} ca_query_proj_params;

/* Low-rank query generation for T tokens (Ch.6 "Low-rank query generation",
 * "The lightning indexer"): from h [T][d] bf16 computes, in two GEMM stages,
 *   c_q [T][d_c]  bf16  = h W^{DQ}            (the shared latent, stored bf16)
 *   w_i [T][n_i]  fp32  = h W^w               (indexer combiner weights)
 *   q   [T][n_q]  bf16  = c_q W^{UQ}          (n_h heads of c, head-major)
 *   q_i [T][n_qi] bf16  = c_q W^{IUQ}         (n_I heads of c_I)
 * q and q_i are the query inputs the indexer and attend calls take.  All
 * outputs are caller-owned device buffers (q_i / w_i may be NULL when n_qi == 0);
 * workspace: ca_query_proj_workspace() bytes of device memory (NULL when 0).
 * Errors: CA_ERR_ARG (NULL pointer, bad sizes, misaligned pointer),
 * CA_ERR_UNSUPPORTED (d or d_c not a multiple of 64), CA_ERR_WORKSPACE. */
size_t ca_query_proj_workspace(const ca_query_proj_params* p, int64_t T);
int ca_query_proj(const ca_query_proj_params* p, const void* h, int64_t T, void* c_q, void* q, void* q_i, float* w_i,
                  void* workspace, size_t workspace_bytes, void* stream);

typedef struct ca_out_proj_params {
  int32_t n_h;        /* query heads; 8 heads a group, g = n_h / 8 groups */
  int32_t c;          /* head width (8 c a multiple of 64) */
  int32_t d_g;        /* width of each group's bottleneck */
  int32_t d;          /* output (hidden) width */
  const void* w_o1;   /* bf16 [g][d_g][8 c]  (group j's projection of heads 8j .. 8j+7) */
  const void* w_o2;   /* bf16 [d][g d_g]     (the concatenated groups to d) */
} ca_out_proj_params;

/* Grouped output projection for T tokens (Ch.6 "Grouped output projections"):
 * o [T][n_h c] bf16 (the attention output, heads concatenated in head order)
 *   u [T][g d_g] bf16: u[:, j d_g .. (j+1) d_g) = o[:, 8 j c .. 8 (j+1) c) W1_j
 *   y [T][d]     bf16 = u W2
 * u and y are caller-owned device buffers; workspace as ca_out_proj_workspace().
 * Errors as ca_query_proj (n_h not a multiple of 8, g d_g not a multiple of 64:
 * CA_ERR_UNSUPPORTED). */
size_t ca_out_proj_workspace(const ca_out_proj_params* p, int64_t T);
int ca_out_proj(const ca_out_proj_params* p, const void* o, int64_t T, void* u, void* y, void* workspace,
                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSAHCA_H */
