// Lightning indexer scores and per-row top-k selection.
//
// dsv4 book Ch.6 "The lightning indexer": I[t,s] = sum_h w[t,h] ReLU(qI[t,h] . K[s])
// over blocks s < floor(t/m) (Ch.5 "Causal availability"); Ch.6 "Top-k selection
// and asymptotic scaling": keep the k best blocks per query.
//
// Scoring is the one real contraction here: for e4m3 keys it runs on the
// gfx950 fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales) with the
// query rows as the A operand (4 queries x 8 heads = 32 rows, or 1 query
// padded for decode) and 32 keys per instruction as the B operand; each lane
// loads 32 contiguous key bytes, so a wavefront streams 2 KB of key codes per
// instruction.  The head combine (weights, ReLU) and the per-key power-of-two
// scales are applied to the fp32 accumulators.
//
// Top-k is exact and deterministic: fp32 scores map to order-preserving
// 32-bit keys (-0 folded onto +0), a 4 x 8-bit radix select finds the k-th
// largest key T and how many keys equal to T are needed, and an ordered
// compaction (ballot prefix counts) emits every key > T plus the lowest-index
// keys == T, in ascending index order.
#include "common.h"
#include "kernels.h"

namespace ca {

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0;                 // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ scores, generic (fp32 math)
// One thread per (row, key).  Query heads for the row sit in LDS (quantized to
// e4m3 first when the pool is e4m3).
__global__ void index_scores_generic_kernel(CacheView cv, int nI, int cI, int m, int q_fmt, const void* qI,
                                            const float* w, const int32_t* pos, int seq_fixed, float* scores,
                                            int64_t stride) {
  extern __shared__ float qs[];                // [nI * cI] query values as the indexer sees them
  const int r = blockIdx.x;
  const int t = pos ? pos[r] : r;
  const int seq = seq_fixed >= 0 ? seq_fixed : r;
  const int64_t ne = t / m < stride ? t / m : stride;   // never beyond the score row
  for (int h = threadIdx.x >> 6; h < nI; h += blockDim.x >> 6) {
    // one wavefront per head: load, optionally quantize exactly like the MFMA path
    int lane = threadIdx.x & 63;
    float amax = 0.0f;
    for (int c = lane; c < cI; c += 64) amax = fmaxf(amax, fabsf(load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + c)));
    amax = wave_max(amax);
    int e = pow2_exponent(amax);
    for (int c = lane; c < cI; c += 64) {
      float v = load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + c);
      if (cv.fmt == CA_E4M3) {
        uint32_t code = e4m3_encode(ldexpf(v, -e));
        v = ldexpf(e4m3x2_to_f32(code)[0], e);
      }
      qs[h * cI + c] = v;
    }
  }
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  if (s >= ne) return;
  uint8_t* page = cv.page_of(seq, s);
  float out = -INFINITY;
  if (page != nullptr) {
    int slot = cv.slot_of(s);
    float acc = 0.0f;
    if (cv.fmt == CA_E4M3) {
      const uint8_t* kp = page + (int64_t)slot * cI;
      float ks = ((const float*)(page + ((int64_t)cI << cv.page_shift)))[slot];
      for (int h = 0; h < nI; ++h) {
        float d = 0.0f;
        for (int c = 0; c < cI; c += 2) {
          f32x2 kv = e4m3x2_to_f32((uint32_t)kp[c] | ((uint32_t)kp[c + 1] << 8));
          d += qs[h * cI + c] * kv[0] + qs[h * cI + c + 1] * kv[1];
        }
        acc += w[(int64_t)r * nI + h] * fmaxf(d * ks, 0.0f);
      }
    } else {
      const float* kp = (const float*)(page + slot * cv.stride);
      for (int h = 0; h < nI; ++h) {
        float d = 0.0f;
        for (int c = 0; c < cI; ++c) d += qs[h * cI + c] * kp[c];
        acc += w[(int64_t)r * nI + h] * fmaxf(d, 0.0f);
      }
    }
    out = acc;
  }
  scores[(int64_t)r * stride + s] = out;
}

// ------------------------------------------------------------------ scores, fp8 MFMA (nI = 8, cI = 64)
// Block: 256 threads (4 waves).  blockIdx.x = group of QPW query rows,
// blockIdx.y = chunk of kScoreChunk keys (64 pages); wave w owns 1,024
// consecutive keys (16 pages) as 32 MFMA blocks of 32 keys, processed in groups
// of 4 blocks with a register double buffer: the loads of group g+1 are in
// flight while group g is scored.  The chunk's slice of the page table is
// staged in LDS once, so key loads never wait on a page-table load.
constexpr int kScoreChunk = 4096;
constexpr int kHistBins = 4096;

struct KeyGroup {
  i32x4 v0[4], v1[4];
  float ks[4];
  bool ok[4];
};

__device__ __forceinline__ void load_key_group(const CacheView& cv, const int* pt_s, int64_t k0, int64_t k1,
                                               int64_t gbase, int lane, KeyGroup& kg) {
  constexpr int cI = 64;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t s = gbase + 32 * u + (lane & 31);
    const int pg = s < k1 ? pt_s[(int)((s - k0) >> cv.page_shift)] : -1;
    kg.ok[u] = pg >= 0;
    kg.v0[u] = i32x4{0, 0, 0, 0};
    kg.v1[u] = kg.v0[u];
    kg.ks[u] = 0.0f;
    if (kg.ok[u]) {
      const uint8_t* base = cv.pool + (int64_t)pg * cv.page_bytes;
      const int slot = cv.slot_of(s);
      const i32x4* kp = (const i32x4*)(base + slot * cI + 32 * (lane >> 5));
      kg.v0[u] = kp[0];
      kg.v1[u] = kp[1];
      kg.ks[u] = ((const float*)(base + (cI << cv.page_shift)))[slot];
    }
  }
}

template <int QPW>
__global__ void __launch_bounds__(256) index_scores_fp8_kernel(CacheView cv, int m, int q_fmt, const void* qI,
                                                               const float* w, const int32_t* pos, int seq_fixed,
                                                               int n_rows, float* scores, int64_t stride) {
  constexpr int nI = 8, cI = 64;
  __shared__ __attribute__((aligned(16))) uint8_t qcodes[32 * cI];  // A operand rows: (query, head)
  __shared__ float wq[32];                                          // w * query scale per row
  __shared__ int pt_s[kScoreChunk / 16];                            // page ids of the chunk (>= 64 pages)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * QPW;

  int64_t ne[QPW];
  int64_t ne_max = 0;
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    int r = r0 + qq;
    int t = r < n_rows ? (pos ? pos[r] : r) : 0;
    ne[qq] = r < n_rows ? (t / m < stride ? t / m : stride) : 0;
    ne_max = ne[qq] > ne_max ? ne[qq] : ne_max;
  }
  const int64_t k0 = (int64_t)blockIdx.y * kScoreChunk;
  if (k0 >= ne_max) return;                            // uniform over the block
  const int64_t k1 = (k0 + kScoreChunk < ne_max) ? k0 + kScoreChunk : ne_max;
  const int seq = seq_fixed >= 0 ? seq_fixed : r0;     // decode: one row per group, row == sequence

  // prologue: the chunk's page ids, and QPW*8 query-head rows quantized to e4m3
  const int n_pg = kScoreChunk >> cv.page_shift;
  for (int i = threadIdx.x; i < n_pg; i += 256) {
    const int64_t pi = (k0 >> cv.page_shift) + i;
    int pg = -1;
    if (pi < cv.max_pages) {
      pg = cv.page_table[(int64_t)seq * cv.max_pages + pi];
      if (pg >= cv.n_pages) pg = -1;
    }
    pt_s[i] = pg;
  }
  for (int row = wave; row < 32; row += 4) {
    int qq = row / nI, hh = row % nI, r = r0 + qq;
    bool valid = qq < QPW && r < n_rows;
    float v = valid ? load_act(qI, q_fmt, ((int64_t)r * nI + hh) * cI + lane) : 0.0f;
    int e = pow2_exponent(wave_max(fabsf(v)));
    qcodes[row * cI + lane] = valid ? (uint8_t)e4m3_encode(ldexpf(v, -e)) : 0;
    if (lane == 0) wq[row] = valid ? w[(int64_t)r * nI + hh] * ldexpf(1.0f, e) : 0.0f;
  }
  __syncthreads();

  // A operand: row lane%32, bytes [32*(lane/32), +32)
  i32x8 a;
  {
    const int* src = (const int*)(qcodes + (lane & 31) * cI + 32 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = src[i];
  }
  float wl[QPW][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq)
#pragma unroll
    for (int v = 0; v < 4; ++v) wl[qq][v] = wq[qq * nI + 4 * (lane >> 5) + v];

  const int64_t wbase = k0 + (kScoreChunk / 4) * wave;
  constexpr int kGroups = kScoreChunk / 4 / 128;       // groups of 4 x 32 keys per wave
  KeyGroup cur, nxt;
  load_key_group(cv, pt_s, k0, k1, wbase, lane, cur);
  for (int grp = 0; grp < kGroups; ++grp) {
    const int64_t gbase = wbase + 128 * grp;
    if (gbase >= k1) break;
    if (grp + 1 < kGroups) load_key_group(cv, pt_s, k0, k1, gbase + 128, lane, nxt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = gbase + 32 * u + (lane & 31);
      const i32x8 bop = __builtin_shufflevector(cur.v0[u], cur.v1[u], 0, 1, 2, 3, 4, 5, 6, 7);
      f32x16 acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, acc, 0, 0, 0, 127, 0, 127);
      // acc[v]: row 8*(v/4) + 4*(lane/32) + v%4 = (query v/4, head 4*(lane/32) + v%4), key lane%32
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float part = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) part += wl[qq][v] * fmaxf(acc[4 * qq + v], 0.0f);
        part += __shfl_xor(part, 32, 64);
        if (lane < 32 && s < ne[qq]) scores[(int64_t)(r0 + qq) * stride + s] = cur.ok[u] ? part * cur.ks[u] : -INFINITY;
      }
    }
    cur = nxt;
  }
}

// ------------------------------------------------------------------ top-k
constexpr int kTopkThreads = 1024;
constexpr int kTopkLdsKeys = 16384;

struct TopkShared {
  uint32_t keys[kTopkLdsKeys];
  uint32_t hist[256];
  uint32_t wsum[kTopkThreads / 64];
  uint32_t wsum2[kTopkThreads / 64];
  uint32_t sel_digit, sel_krem;
};

__device__ __forceinline__ uint32_t get_key(const TopkShared& sh, bool in_lds, const float* row, int64_t s) {
  return in_lds ? sh.keys[s] : order_key(row[s]);
}

// Exclusive prefix of 0/1 flags over the block (index order = thread order).
// Returns the prefix for this thread; *total receives the block total.
__device__ __forceinline__ uint32_t block_flag_prefix(bool f, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t b = __ballot(f);
  uint32_t in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(b);
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    uint32_t c = wsum[i];
    before += i < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

__global__ void __launch_bounds__(kTopkThreads) topk_rows_kernel(const float* scores, int64_t stride,
                                                                 const int32_t* pos, int m, int k, int32_t* out_idx,
                                                                 int32_t* out_cnt, float* out_score) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int t = pos ? pos[r] : r;
  const int64_t n = t / m < stride ? t / m : stride;
  const float* row = scores + (int64_t)r * stride;
  int32_t* oi = out_idx + (int64_t)r * k;
  float* os = out_score ? out_score + (int64_t)r * k : nullptr;
  const int tid = threadIdx.x;

  if (n <= k) {  // every eligible block is kept
    for (int j = tid; j < k; j += blockDim.x) {
      oi[j] = j < n ? j : -1;
      if (os) os[j] = j < n ? row[j] : -INFINITY;
    }
    if (tid == 0) out_cnt[r] = (int32_t)n;
    return;
  }
  const bool in_lds = n <= kTopkLdsKeys;
  if (in_lds)
    for (int64_t s = tid; s < n; s += blockDim.x) sh.keys[s] = order_key(row[s]);

  uint32_t prefix = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += blockDim.x) {
      uint32_t key = get_key(sh, in_lds, row, s);
      if ((key & hi_mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns digits 4L..4L+3; suffix counts from the top digit down
      uint32_t c0 = sh.hist[4 * tid], c1 = sh.hist[4 * tid + 1], c2 = sh.hist[4 * tid + 2], c3 = sh.hist[4 * tid + 3];
      uint32_t lsum = c0 + c1 + c2 + c3;
      uint32_t incl = lsum;  // inclusive suffix sum over lanes >= tid
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_down(incl, o, 64);
        if (tid + o < 64) incl += v;
      }
      uint32_t suffix_above = incl - lsum;
      uint32_t cnts[4] = {c0, c1, c2, c3};
      uint32_t cum = suffix_above;  // keys with digit > 4*tid+3
      for (int d = 3; d >= 0; --d) {
        uint32_t nc = cum + cnts[d];
        if (cum < krem && nc >= krem) {
          sh.sel_digit = 4 * tid + d;
          sh.sel_krem = krem - cum;
        }
        cum = nc;
      }
    }
    __syncthreads();
    prefix |= sh.sel_digit << shift;
    krem = sh.sel_krem;
    __syncthreads();
  }
  // prefix == T (the k-th largest key); krem == how many keys equal to T to keep
  const uint32_t T = prefix, need_eq = krem;
  uint32_t eq_seen = 0, taken = 0;
  for (int64_t base = 0; base < n; base += blockDim.x) {
    int64_t s = base + tid;
    uint32_t key = s < n ? get_key(sh, in_lds, row, s) : 0u;
    bool gt = s < n && key > T, eq = s < n && key == T;
    uint32_t eq_tot, tk_tot;
    uint32_t eq_rank = eq_seen + block_flag_prefix(eq, sh.wsum, &eq_tot);
    bool take = gt || (eq && eq_rank < need_eq);
    uint32_t o = taken + block_flag_prefix(take, sh.wsum2, &tk_tot);
    if (take && o < (uint32_t)k) {
      oi[o] = (int32_t)s;
      if (os) os[o] = row[s];
    }
    eq_seen += eq_tot;
    taken += tk_tot;
  }
  if (tid == 0) out_cnt[r] = k;
}

// ------------------------------------------------------------------ top-k, long rows (decode)
// Rows with more candidates than one workgroup should stream (decode at long
// context: 262,144 per row at 2^20 tokens) are selected in three passes that
// spread the scan over many workgroups:
//   1. histogram of the top 12 key bits per row (LDS histogram per chunk,
//      nonzero bins added to the row's global histogram: integer atomics, so
//      the counts are order independent);
//   2. every chunk finds the bin b* holding the k-th largest key from the row
//      histogram and appends its keys with bin >= b* (about k plus one bin's
//      population) to a per-row candidate list;
//   3. one workgroup per row selects exactly among the candidates (radix select
//      on the full key, then the lowest indices among keys equal to the
//      threshold) and sorts the kept indices ascending.
// The candidate list is filled in arbitrary order, but pass 3 depends only on
// the set of (key, index) pairs, so the result is deterministic.
constexpr int kChunk = 4096;
constexpr int kResolveThreads = 1024;
constexpr int kResolveLds = 8192;     // candidates held in LDS (more spill to the global list)
constexpr int kSortMax = 8192;        // largest k the resolve pass sorts in LDS

__global__ void topk_zero_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__device__ __forceinline__ int64_t row_len(const int32_t* pos, int r, int m, int64_t stride) {
  int t = pos ? pos[r] : r;
  int64_t n = t / m;
  return n < stride ? n : stride;
}

__global__ void __launch_bounds__(256) topk_hist_kernel(const float* scores, int64_t stride, const int32_t* pos,
                                                        int m, int k, uint32_t* hist) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)r * stride;
  const int64_t c1 = c0 + kChunk < n ? c0 + kChunk : n;
  for (int64_t s = c0 + threadIdx.x; s < c1; s += blockDim.x) atomicAdd(&h[order_key(row[s]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = hist + (int64_t)r * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

// Bin holding the k-th largest key of a row, from its histogram (block of 256
// threads): the histogram is staged in LDS, each thread sums 16 bins, wave 0
// finds the thread whose bins hold the k-th key by a suffix scan, and that
// thread walks its 16 bins from the top.
__device__ uint32_t threshold_bin(const uint32_t* g, int k, uint32_t* hb, uint32_t* part) {
  __shared__ uint32_t sel_owner, sel_above, sel_bin;
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += 256) hb[i] = g[i];
  __syncthreads();
  uint32_t sum = 0;
  for (int i = 0; i < 16; ++i) sum += hb[16 * tid + i];
  part[tid] = sum;
  __syncthreads();
  if (tid < 64) {
    // lane L owns threads 4L..4L+3; suffix sums from the top thread down
    uint32_t c[4] = {part[4 * tid], part[4 * tid + 1], part[4 * tid + 2], part[4 * tid + 3]};
    uint32_t lsum = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = lsum;
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t v = __shfl_down(incl, o, 64);
      if (tid + o < 64) incl += v;
    }
    uint32_t cum = incl - lsum;
    for (int d = 3; d >= 0; --d) {
      uint32_t nxt = cum + c[d];
      if (cum < (uint32_t)k && nxt >= (uint32_t)k) {
        sel_owner = 4 * tid + d;
        sel_above = cum;
      }
      cum = nxt;
    }
  }
  __syncthreads();
  if (tid == (int)sel_owner) {
    uint32_t cum = sel_above;
    for (int b = 16 * tid + 15; b >= 16 * tid; --b) {
      if (cum + hb[b] >= (uint32_t)k) {
        sel_bin = (uint32_t)b;
        break;
      }
      cum += hb[b];
    }
  }
  __syncthreads();
  return sel_bin;
}

__global__ void __launch_bounds__(256) topk_gather_kernel(const float* scores, int64_t stride, const int32_t* pos,
                                                          int m, int k, const uint32_t* hist, uint32_t* cand_n,
                                                          uint32_t* cand_key, uint32_t* cand_idx) {
  __shared__ uint32_t part[256];
  __shared__ uint32_t hb[kHistBins];
  __shared__ uint32_t base_s;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  const uint32_t bstar = threshold_bin(hist + (int64_t)r * kHistBins, k, hb, part);
  const float* row = scores + (int64_t)r * stride;
  // each thread owns 16 consecutive keys of the chunk
  constexpr int kPer = kChunk / 256;
  const int64_t s0 = c0 + (int64_t)tid * kPer;
  uint32_t keys[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t s = s0 + i;
    keys[i] = s < n ? order_key(row[s]) : 0u;
    mine += (s < n && (keys[i] >> 20) >= bstar) ? 1u : 0u;
  }
  // block-wide exclusive prefix of the per-thread counts, one reservation per block
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t incl = mine;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  __syncthreads();
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  uint32_t before = incl - mine, total = 0;
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? part[w] : 0u;
    total += part[w];
  }
  if (tid == 0) base_s = total ? atomicAdd(&cand_n[r], total) : 0u;
  __syncthreads();
  uint32_t o = base_s + before;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t s = s0 + i;
    if (s < n && (keys[i] >> 20) >= bstar) {
      cand_key[(int64_t)r * stride + o] = keys[i];
      cand_idx[(int64_t)r * stride + o] = (uint32_t)s;
      ++o;
    }
  }
}

struct ResolveShared {
  uint32_t key[kResolveLds];
  uint32_t idx[kResolveLds];
  uint32_t hist[256];
  uint32_t wsum[kResolveThreads / 64];
  uint32_t sel_digit, sel_krem, n_eq, n_out;
};

// In-LDS bitonic sort (ascending) of n_pow2 32-bit values.
__device__ void bitonic_sort(uint32_t* v, int n_pow2) {
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n_pow2 / 2; i += blockDim.x) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = (lo & size) == 0;
        uint32_t a = v[lo], b = v[hi];
        if ((a > b) == up) {
          v[lo] = b;
          v[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kResolveThreads) topk_resolve_kernel(const float* scores, int64_t stride,
                                                                       const int32_t* pos, int m, int k,
                                                                       const uint32_t* cand_n,
                                                                       const uint32_t* cand_key,
                                                                       const uint32_t* cand_idx, int32_t* out_idx,
                                                                       int32_t* out_cnt, float* out_score) {
  __shared__ ResolveShared sh;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const float* row = scores + (int64_t)r * stride;
  int32_t* oi = out_idx + (int64_t)r * k;
  float* os = out_score ? out_score + (int64_t)r * k : nullptr;
  if (n <= k) {
    for (int j = tid; j < k; j += blockDim.x) {
      oi[j] = j < n ? j : -1;
      if (os) os[j] = j < n ? row[j] : -INFINITY;
    }
    if (tid == 0) out_cnt[r] = (int32_t)n;
    return;
  }
  const uint32_t nc = cand_n[r];
  const bool in_lds = nc <= (uint32_t)kResolveLds;
  const uint32_t* gk = cand_key + (int64_t)r * stride;
  const uint32_t* gi = cand_idx + (int64_t)r * stride;
  if (in_lds)
    for (uint32_t i = tid; i < nc; i += blockDim.x) {
      sh.key[i] = gk[i];
      sh.idx[i] = gi[i];
    }
  // radix select of the k-th largest key among the candidates
  uint32_t prefix = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nc; i += blockDim.x) {
      uint32_t key = in_lds ? sh.key[i] : gk[i];
      if ((key & hi_mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c[4] = {sh.hist[4 * tid], sh.hist[4 * tid + 1], sh.hist[4 * tid + 2], sh.hist[4 * tid + 3]};
      uint32_t lsum = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = lsum;
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_down(incl, o, 64);
        if (tid + o < 64) incl += v;
      }
      uint32_t cum = incl - lsum;
      for (int d = 3; d >= 0; --d) {
        uint32_t nxt = cum + c[d];
        if (cum < krem && nxt >= krem) {
          sh.sel_digit = 4 * tid + d;
          sh.sel_krem = krem - cum;
        }
        cum = nxt;
      }
    }
    __syncthreads();
    prefix |= sh.sel_digit << shift;
    krem = sh.sel_krem;
    __syncthreads();
  }
  const uint32_t T = prefix, need_eq = krem;
  // kept set: every candidate above T, then the need_eq lowest indices equal to T.
  // sh.idx is reused as the output buffer once the candidates are consumed from wherever they live.
  __shared__ uint32_t outbuf[kSortMax];
  __shared__ uint32_t eqbuf[kSortMax];
  if (tid == 0) {
    sh.n_eq = 0;
    sh.n_out = 0;
  }
  __syncthreads();
  for (uint32_t i = tid; i < nc; i += blockDim.x) {
    uint32_t key = in_lds ? sh.key[i] : gk[i];
    uint32_t id = in_lds ? sh.idx[i] : gi[i];
    if (key > T) {
      uint32_t o = atomicAdd(&sh.n_out, 1u);
      if (o < (uint32_t)kSortMax) outbuf[o] = id;
    } else if (key == T) {
      uint32_t o = atomicAdd(&sh.n_eq, 1u);
      if (o < (uint32_t)kSortMax) eqbuf[o] = id;
    }
  }
  __syncthreads();
  const uint32_t n_gt = sh.n_out, n_eq = sh.n_eq;
  if (n_eq <= (uint32_t)kSortMax) {
    int p2 = 1;
    while (p2 < (int)n_eq) p2 <<= 1;
    for (int i = (int)n_eq + tid; i < p2; i += blockDim.x) eqbuf[i] = 0xFFFFFFFFu;
    __syncthreads();
    bitonic_sort(eqbuf, p2);
    for (uint32_t j = tid; j < need_eq; j += blockDim.x) outbuf[n_gt + j] = eqbuf[j];
  } else {
    // pathological tie count: take the need_eq smallest equal indices one at a time
    __shared__ uint32_t last, best;
    if (tid == 0) last = 0xFFFFFFFFu;
    __syncthreads();
    for (uint32_t j = 0; j < need_eq; ++j) {
      if (tid == 0) best = 0xFFFFFFFFu;
      __syncthreads();
      uint32_t mine = 0xFFFFFFFFu;
      for (uint32_t i = tid; i < nc; i += blockDim.x) {
        uint32_t key = in_lds ? sh.key[i] : gk[i];
        uint32_t id = in_lds ? sh.idx[i] : gi[i];
        if (key == T && (last == 0xFFFFFFFFu || id > last) && id < mine) mine = id;
      }
      atomicMin(&best, mine);
      __syncthreads();
      if (tid == 0) {
        outbuf[n_gt + j] = best;
        last = best;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  int p2 = 1;
  while (p2 < k) p2 <<= 1;
  for (int i = k + tid; i < p2; i += blockDim.x) outbuf[i] = 0xFFFFFFFFu;
  __syncthreads();
  bitonic_sort(outbuf, p2);
  for (int j = tid; j < k; j += blockDim.x) {
    uint32_t id = outbuf[j];
    oi[j] = (int32_t)id;
    if (os) os[j] = row[id];
  }
  if (tid == 0) out_cnt[r] = k;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_index_scores(const CacheView& cv, const ca_index_params& p, const void* qI, const float* w,
                               const int32_t* pos, int seq_fixed, int n_rows, int64_t max_pos, float* scores,
                               int64_t stride, void* ws_long, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  int64_t max_ne = max_pos / p.ratio;
  if (max_ne == 0) return hipSuccess;
  const bool long_rows = ws_long != nullptr && topk_use_long(stride, p.k);
  uint32_t* hist = long_rows ? (uint32_t*)ws_long : nullptr;
  if (long_rows) {  // clear the histograms and candidate counters of the multi-workgroup top-k
    const int64_t nz = (int64_t)n_rows * (kHistBins + 1);
    hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, hist, nz);
  }
  if (cv.fmt == CA_E4M3 && p.n_heads == 8 && p.dim == 64 && cv.page_shift >= 4) {
    const int64_t chunks = (max_ne + kScoreChunk - 1) / kScoreChunk;
    if (seq_fixed >= 0) {
      dim3 grid((unsigned)((n_rows + 3) / 4), (unsigned)chunks);
      hipLaunchKernelGGL(index_scores_fp8_kernel<4>, grid, dim3(256), 0, st, cv, p.ratio, p.q_format, qI, w, pos,
                         seq_fixed, n_rows, scores, stride);
    } else {
      dim3 grid((unsigned)n_rows, (unsigned)chunks);
      hipLaunchKernelGGL(index_scores_fp8_kernel<1>, grid, dim3(256), 0, st, cv, p.ratio, p.q_format, qI, w, pos,
                         seq_fixed, n_rows, scores, stride);
    }
  } else {
    dim3 grid((unsigned)n_rows, (unsigned)((max_ne + 255) / 256));
    size_t sm = sizeof(float) * p.n_heads * p.dim;
    hipLaunchKernelGGL(index_scores_generic_kernel, grid, dim3(256), sm, st, cv, p.n_heads, p.dim, p.ratio,
                       p.q_format, qI, w, pos, seq_fixed, scores, stride);
  }
  if (hist != nullptr) {  // scores written without a fused histogram: count them now
    const unsigned chunks = (unsigned)((stride + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(n_rows, chunks), dim3(256), 0, st, scores, stride, pos, p.ratio, p.k,
                       hist);
  }
  return hipGetLastError();
}

size_t topk_long_workspace(int n_rows, int64_t stride) {
  return (size_t)n_rows * kHistBins * 4 + (size_t)n_rows * 4 + 2 * (size_t)n_rows * stride * 4 + 256;
}

bool topk_use_long(int64_t stride, int k) { return stride > kTopkLdsKeys && k <= kSortMax; }

hipError_t launch_topk(const float* scores, int64_t stride, const int32_t* pos, int m, int k, int n_rows,
                       int32_t* out_idx, int32_t* out_cnt, float* out_score, void* ws_long, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  if (ws_long != nullptr && topk_use_long(stride, k)) {
    uint32_t* hist = (uint32_t*)ws_long;
    uint32_t* cand_n = hist + (int64_t)n_rows * kHistBins;
    uint32_t* cand_key = cand_n + n_rows;
    uint32_t* cand_idx = cand_key + (int64_t)n_rows * stride;
    // the histogram was filled by the scoring launch (see launch_index_scores)
    const unsigned chunks = (unsigned)((stride + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(topk_gather_kernel, dim3(n_rows, chunks), dim3(256), 0, st, scores, stride, pos, m, k, hist,
                       cand_n, cand_key, cand_idx);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(n_rows), dim3(kResolveThreads), 0, st, scores, stride, pos, m, k,
                       cand_n, cand_key, cand_idx, out_idx, out_cnt, out_score);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_rows_kernel, dim3(n_rows), dim3(kTopkThreads), 0, st, scores, stride,
                     pos, m, k, out_idx, out_cnt, out_score);
  return hipGetLastError();
}

}  // namespace ca
