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
// scales are applied to the fp32 accumulators.  FP4 keys (dsv4 book Ch.8: e2m1
// with a 1-byte scale per 32 elements) use the same instruction with e2m1 B
// operands, whose E8M0 block scales the instruction applies itself.
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
// One thread per (row, key).  Query heads for the row sit in LDS (quantized first
// when the pool is e4m3 or FP4: to e4m3 per head, or with q_fp4 to FP4 per
// 32-channel block).
__global__ void index_scores_generic_kernel(CacheView cv, int nI, int cI, int m, int q_fmt, const void* qI,
                                            const float* w, RowPos pos, int seq_fixed, float* scores,
                                            int64_t stride, int q_fp4) {
  extern __shared__ float qs[];                // [nI * cI] query values as the indexer sees them
  const int r = blockIdx.x;
  const int t = pos(r);
  const int seq = seq_fixed >= 0 ? seq_fixed : r;
  const int64_t ne = t / m < stride ? t / m : stride;   // never beyond the score row
  for (int h = threadIdx.x >> 6; h < nI; h += blockDim.x >> 6) {
    // one wavefront per head: load, optionally quantize exactly like the MFMA path
    int lane = threadIdx.x & 63;
    if (q_fp4) {   // (uniform) 32-channel blocks are the wavefront's halves (c_I % 32 == 0)
      for (int c0 = 0; c0 < cI; c0 += 64) {
        const int c = c0 + lane;
        const float v = c < cI ? load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + c) : 0.0f;
        float bmax = fabsf(v);
        for (int o = 16; o > 0; o >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o, 64));
        const int e = fp4_block_exponent(bmax);
        if (c < cI) qs[h * cI + c] = ldexpf(e2m1_to_f32(e2m1_encode(ldexpf(v, -e))), e);
      }
      continue;
    }
    float amax = 0.0f;
    for (int c = lane; c < cI; c += 64) amax = fmaxf(amax, fabsf(load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + c)));
    amax = wave_max(amax);
    int e = pow2_exponent(amax);
    for (int c = lane; c < cI; c += 64) {
      float v = load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + c);
      if (cv.fmt == CA_E4M3 || cv.fmt == CA_FP4) {
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
    } else if (cv.fmt == CA_FP4) {
      const uint8_t* kp = page + (int64_t)slot * (cI / 2);
      const uint8_t* sp = page + ((int64_t)(cI / 2) << cv.page_shift) + (int64_t)slot * (cI / 32);
      for (int h = 0; h < nI; ++h) {
        float d = 0.0f;
        for (int b = 0; b < cI / 32; ++b) {
          float db = 0.0f;
          for (int c = 32 * b; c < 32 * b + 32; c += 2) {
            const uint32_t byte = kp[c >> 1];
            db += qs[h * cI + c] * e2m1_to_f32(byte & 15u) + qs[h * cI + c + 1] * e2m1_to_f32(byte >> 4);
          }
          d += ldexpf(db, (int)sp[b] - 127);
        }
        acc += w[(int64_t)r * nI + h] * fmaxf(d, 0.0f);
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
// of G blocks with a register double buffer: the loads of group g+1
// are in flight while group g is scored.  The chunk's slice of the page table is
// staged in LDS once, so key loads never wait on a page-table load.
constexpr int kScoreChunk = 4096;
constexpr int kHistBins = 4096;

// MFMA blocks of 32 keys per load group (and per buffer), for either key format
// (16 for FP4 keys measured slower: fewer waves per SIMD)
template <int KF> constexpr int group_blocks() { return 8; }

template <int G>
struct KeyGroup {
  i32x4 v0[G], v1[G];   // e4m3: 32 code bytes; FP4: v0 = 16 code bytes
  float ks[G];          // e4m3: the key's scale
  int sc[G];            // FP4: the E8M0 byte of the lane's 32-channel block
  bool ok[G];
};

// Loads of a group of G MFMA blocks of 32 keys (key = lane % 32 of each).
// e4m3 pages: lane half h takes the key's code bytes [32h, 32h + 32).  FP4 pages:
// lane half h takes the bytes [16h, 16h + 16) (channels 32h .. 32h + 31) and the
// E8M0 byte of block h.
template <int KF, int G>
__device__ __forceinline__ void load_key_group(const CacheView& cv, const int* pt_s, int64_t k0, int64_t k1,
                                               int64_t gbase, int lane, KeyGroup<G>& kg) {
  constexpr int cI = 64;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int64_t s = gbase + 32 * u + (lane & 31);
    const int pg = s < k1 ? pt_s[(int)((s - k0) >> cv.page_shift)] : -1;
    kg.ok[u] = pg >= 0;
    kg.v0[u] = i32x4{0, 0, 0, 0};
    kg.v1[u] = kg.v0[u];
    kg.ks[u] = 0.0f;
    kg.sc[u] = 127;
    if (kg.ok[u]) {
      const uint8_t* base = cv.pool + (int64_t)pg * cv.page_bytes;
      const int slot = cv.slot_of(s);
      if constexpr (KF == CA_FP4) {
        kg.v0[u] = *(const i32x4*)(base + slot * (cI / 2) + 16 * (lane >> 5));
        kg.sc[u] = base[((cI / 2) << cv.page_shift) + slot * (cI / 32) + (lane >> 5)];
      } else {
        const i32x4* kp = (const i32x4*)(base + slot * cI + 32 * (lane >> 5));
        kg.v0[u] = kp[0];
        kg.v1[u] = kp[1];
        kg.ks[u] = ((const float*)(base + (cI << cv.page_shift)))[slot];
      }
    }
  }
}

// KF: key page format, CA_E4M3 (fp8 x fp8 products, the key's scale applied to
// the accumulator) or CA_FP4 (fp8 queries x e2m1 keys with the E8M0 block scales
// applied by the MFMA).  The e2m1 operand of the 32x32x64 MFMA holds, in lane
// half h, K = 32h .. 32h + 31; the e4m3 operand facing it holds, in lane half h,
// the 16 bytes of K = 16h .. 16h + 15 then those of K = 32 + 16h .. +15 (layout
// measured on the device).  e4m3 x e4m3 products only need the same order on
// both sides, which the plain 32-byte halves give.
// QF: query format, CA_E4M3 (one power-of-two scale per (query, head), folded
// into w) or CA_FP4 (FP4 keys only: e2m1 codes with one E8M0 byte per 32
// channels, applied by the MFMA as the A scale; an e2m1 A operand holds, in lane
// half h, K = 32h .. 32h + 31 like the B operand, measured on the device).
// hist (QPW == 1 only, else null): the row's long-top-k state, already zeroed;
// when the row has more than hist_k keys, the workgroup adds the histogram of its
// chunk's scores (top 12 bits of the order-preserving keys) to it, from an LDS
// histogram in dynamic shared memory (kHistBins words).
template <int QPW, int KF, int QF>
__device__ __forceinline__ void index_scores_mfma(CacheView cv, int m, int q_fmt, const void* qI, const float* w,
                                                  RowPos pos, int seq_fixed, int n_rows, float* scores,
                                                  int64_t stride, uint32_t* hist, int hist_words, int hist_k) {
  static_assert(QF == CA_E4M3 || (QF == CA_FP4 && KF == CA_FP4), "FP4 queries meet FP4 keys");
  constexpr int nI = 8, cI = 64;
  constexpr int kQBytes = QF == CA_FP4 ? cI / 2 : cI;              // code bytes per query-head row
  extern __shared__ uint32_t hs[];
  __shared__ __attribute__((aligned(16))) uint8_t qcodes[32 * cI];  // A operand rows: (query, head)
  __shared__ uint8_t qsc[32][2];                                    // FP4 queries: E8M0 byte per block
  __shared__ float wq[32];                                          // w (* query scale for e4m3) per row
  __shared__ int pt_s[kScoreChunk / 16];                            // page ids of the chunk (>= 64 pages)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * QPW;

  const int seq = seq_fixed >= 0 ? seq_fixed : r0;     // decode: one row per group, row == sequence
  const int64_t k0 = (int64_t)blockIdx.y * kScoreChunk;

  // The loads that do not depend on the row positions go out first: the chunk's page
  // ids (one per thread: n_pg <= 256 pages as page_shift >= 4) and the query rows.
  const int n_pg = kScoreChunk >> cv.page_shift;
  int pg = -1;
  if (threadIdx.x < n_pg) {
    const int64_t pi = (k0 >> cv.page_shift) + threadIdx.x;
    if (pi < cv.max_pages) pg = cv.page_table[(int64_t)seq * cv.max_pages + pi];
  }
  constexpr int kRowsPerWave = 32 / 4;                 // query-head rows (query, head) of each wave
  float qv[kRowsPerWave];
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int row = wave + 4 * j, qq = row / nI, h = row % nI, r = r0 + qq;
    qv[j] = (qq < QPW && r < n_rows) ? load_act(qI, q_fmt, ((int64_t)r * nI + h) * cI + lane) : 0.0f;
  }

  int64_t ne[QPW];
  int64_t ne_max = 0;
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    int r = r0 + qq;
    int t = r < n_rows ? pos(r) : 0;
    ne[qq] = r < n_rows ? (t / m < stride ? t / m : stride) : 0;
    ne_max = ne[qq] > ne_max ? ne[qq] : ne_max;
  }
  if (k0 >= ne_max) return;                            // uniform over the block
  const bool want_hist = QPW == 1 && hist != nullptr && ne[0] > hist_k;   // uniform
  if (want_hist)
    for (int i = threadIdx.x; i < kHistBins; i += 256) hs[i] = 0u;
  const int64_t k1 = (k0 + kScoreChunk < ne_max) ? k0 + kScoreChunk : ne_max;

  // prologue: the chunk's page ids into LDS, and QPW*8 query-head rows quantized to e4m3
  if (threadIdx.x < n_pg) pt_s[threadIdx.x] = pg < cv.n_pages ? pg : -1;
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int row = wave + 4 * j, qq = row / nI, h = row % nI, r = r0 + qq;
    if (qq < QPW && r < n_rows) {                      // (uniform) rows past the group's queries stay zero
      const float v = qv[j];
      if constexpr (QF == CA_FP4) {
        // the 32-channel blocks are the wavefront's halves: block maximum, exponent,
        // then channel pairs (2c, 2c+1) packed into byte c, low nibble first
        float amax = fabsf(v);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const int e = fp4_block_exponent(amax);
        const uint32_t code = e2m1_encode(ldexpf(v, -e));
        const uint32_t odd = __shfl_xor(code, 1, 64);
        if ((lane & 1) == 0) qcodes[row * kQBytes + (lane >> 1)] = (uint8_t)(code | (odd << 4));
        if ((lane & 31) == 0) qsc[row][lane >> 5] = (uint8_t)(e + 127);
        if (lane == 0) wq[row] = w[(int64_t)r * nI + h];
      } else {
        const int e = pow2_exponent(wave_max(fabsf(v)));
        qcodes[row * cI + lane] = (uint8_t)e4m3_encode(ldexpf(v, -e));
        if (lane == 0) wq[row] = w[(int64_t)r * nI + h] * ldexpf(1.0f, e);
      }
    } else {
      if (lane < kQBytes) qcodes[row * kQBytes + lane] = 0;
      if (lane < 2) qsc[row][lane] = 127;
      if (lane == 0) wq[row] = 0.0f;
    }
  }
  __syncthreads();

  // A operand: row lane%32.  e4m3 queries, e4m3 keys: bytes [32*(lane/32), +32);
  // e4m3 queries, FP4 keys: bytes [16*(lane/32), +16) then [32 + 16*(lane/32), +16);
  // FP4 queries: the 16 code bytes [16*(lane/32), +16) and the block's scale byte
  i32x8 a;
  int a_scale = 127;
  if constexpr (QF == CA_FP4) {
    const int* src = (const int*)(qcodes + (lane & 31) * kQBytes + 16 * (lane >> 5));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = src[i];
      a[4 + i] = 0;
    }
    a_scale = qsc[lane & 31][lane >> 5];
  } else {
    const uint8_t* qrow = qcodes + (lane & 31) * cI;
    const int* src0 = (const int*)(qrow + (KF == CA_FP4 ? 16 : 32) * (lane >> 5));
    const int* src1 = (const int*)(qrow + (KF == CA_FP4 ? 32 + 16 * (lane >> 5) : 32 * (lane >> 5) + 16));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = src0[i];
      a[4 + i] = src1[i];
    }
  }
  float wl[QPW][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq)
#pragma unroll
    for (int v = 0; v < 4; ++v) wl[qq][v] = wq[qq * nI + 4 * (lane >> 5) + v];

  const int64_t wbase = k0 + (kScoreChunk / 4) * wave;
  constexpr int G = group_blocks<KF>();
  constexpr int kGroupKeys = 32 * G;
  constexpr int kGroups = kScoreChunk / 4 / kGroupKeys;  // groups per wave
  KeyGroup<G> cur, nxt;
  load_key_group<KF, G>(cv, pt_s, k0, k1, wbase, lane, cur);
  for (int grp = 0; grp < kGroups; ++grp) {
    const int64_t gbase = wbase + kGroupKeys * grp;
    if (gbase >= k1) break;
    if (grp + 1 < kGroups) load_key_group<KF, G>(cv, pt_s, k0, k1, gbase + kGroupKeys, lane, nxt);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t s = gbase + 32 * u + (lane & 31);
      const i32x8 bop = __builtin_shufflevector(cur.v0[u], cur.v1[u], 0, 1, 2, 3, 4, 5, 6, 7);
      f32x16 acc = {};
      if constexpr (QF == CA_FP4)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, acc, 4, 4, 0, a_scale, 0, cur.sc[u]);
      else if constexpr (KF == CA_FP4)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, acc, 0, 4, 0, 127, 0, cur.sc[u]);
      else
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, acc, 0, 0, 0, 127, 0, 127);
      // acc[v]: row 8*(v/4) + 4*(lane/32) + v%4 = (query v/4, head 4*(lane/32) + v%4), key lane%32
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float part = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) part += wl[qq][v] * fmaxf(acc[4 * qq + v], 0.0f);
        part += __shfl_xor(part, 32, 64);
        if (lane < 32 && s < ne[qq]) {
          const float sc = cur.ok[u] ? (KF == CA_FP4 ? part : part * cur.ks[u]) : -INFINITY;
          scores[(int64_t)(r0 + qq) * stride + s] = sc;
          if (want_hist) atomicAdd(&hs[order_key(sc) >> 20], 1u);
        }
      }
    }
    cur = nxt;
  }
  if (want_hist) {   // the chunk's nonzero bins into the row's histogram (integer adds: order free)
    __syncthreads();
    uint32_t* g = hist + (int64_t)r0 * hist_words;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t c = hs[i];
      if (c) atomicAdd(&g[i], c);
    }
  }
}

// e4m3 queries against e4m3 or FP4 keys
template <int QPW, int KF>
__global__ void __launch_bounds__(256) index_scores_fp8_kernel(CacheView cv, int m, int q_fmt, const void* qI,
                                                               const float* w, RowPos pos, int seq_fixed,
                                                               int n_rows, float* scores, int64_t stride,
                                                               uint32_t* hist, int hist_words, int hist_k) {
  index_scores_mfma<QPW, KF, CA_E4M3>(cv, m, q_fmt, qI, w, pos, seq_fixed, n_rows, scores, stride, hist, hist_words,
                                      hist_k);
}

// FP4 queries against FP4 keys
template <int QPW>
__global__ void __launch_bounds__(256) index_scores_fp4_kernel(CacheView cv, int m, int q_fmt, const void* qI,
                                                               const float* w, RowPos pos, int seq_fixed,
                                                               int n_rows, float* scores, int64_t stride,
                                                               uint32_t* hist, int hist_words, int hist_k) {
  index_scores_mfma<QPW, CA_FP4, CA_FP4>(cv, m, q_fmt, qI, w, pos, seq_fixed, n_rows, scores, stride, hist,
                                         hist_words, hist_k);
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
                                                                 RowPos pos, int m, int k, int32_t* out_idx,
                                                                 int32_t* out_cnt, float* out_score) {
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int t = pos(r);
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
//      nonzero bins added to the row's global histogram with integer atomics, so
//      the counts are order independent), made by the scoring kernel itself when
//      it runs one row per workgroup, else by a pass of its own;
//   2. every chunk finds, from the row's histogram, the bin b* holding the k-th
//      largest key (and the number of keys above it), then appends its keys with
//      bin >= b* to a per-row candidate list;
//   3. one workgroup per row finishes the select among the candidates: two 10-bit
//      radix passes over the keys in bin b* give the exact threshold key T, then
//      the kept indices (every key above T, and the lowest-indexed keys equal to
//      T) are set in LDS bitmaps that are read out in index order.
// The candidate list is filled in arbitrary order, but pass 3 depends only on
// the set of (key, index) pairs, so the result is deterministic.
constexpr int kChunk = 4096;
constexpr int kResolveThreads = 1024;
constexpr int kSortMax = 8192;        // largest k of the long path
constexpr int kMetaWords = 4;         // per row: candidates appended, (spare), b*, keys above b*
constexpr int kRowWords = kHistBins + kMetaWords;   // per-row state: histogram, then the counters
static_assert(kRowWords == kTopkRowWords, "per-row long top-k state size");
constexpr int kRegCand = 4;            // candidates per resolve thread held in registers
constexpr int kBitmapLdsWords = 16384;  // two LDS bitmaps of rows up to 262,144 keys (larger rows: workspace)

__global__ void topk_zero_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__device__ __forceinline__ int64_t row_len(RowPos pos, int r, int m, int64_t stride) {
  int t = pos(r);
  int64_t n = t / m;
  return n < stride ? n : stride;
}

// Bin of a 256-thread block's histogram hb[kHistBins] (in LDS) holding the k-th
// largest key, and the number of keys in higher bins: each thread sums 16 bins,
// wave 0 finds the thread whose bins hold the k-th key by a suffix scan, and that
// thread walks its 16 bins from the top.
__device__ void threshold_bin(const uint32_t* hb, int k, uint32_t* part, uint32_t* bin, uint32_t* above) {
  __shared__ uint32_t sel_owner, sel_above, sel_bin, sel_cum;
  const int tid = threadIdx.x;
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
        sel_cum = cum;
        break;
      }
      cum += hb[b];
    }
  }
  __syncthreads();
  *bin = sel_bin;
  *above = sel_cum;
}

__global__ void __launch_bounds__(256) topk_hist_kernel(const float* scores, int64_t stride, RowPos pos,
                                                        int m, int k, uint32_t* state) {
  __shared__ uint32_t h[kHistBins];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  for (int i = tid; i < kHistBins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)r * stride;
  const int64_t c1 = c0 + kChunk < n ? c0 + kChunk : n;
  for (int64_t s = c0 + tid; s < c1; s += blockDim.x) atomicAdd(&h[order_key(row[s]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = state + (int64_t)r * kRowWords;
  for (int i = tid; i < kHistBins; i += blockDim.x)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

__global__ void __launch_bounds__(256) topk_gather_kernel(const float* scores, int64_t stride, RowPos pos,
                                                          int m, int k, uint32_t* state, uint32_t* cand_key,
                                                          uint32_t* cand_idx) {
  __shared__ uint32_t part[4];
  __shared__ uint32_t base_s;
  __shared__ uint32_t hb[kHistBins];
  __shared__ uint32_t hpart[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  uint32_t* g = state + (int64_t)r * kRowWords;
  uint32_t* meta = g + kHistBins;
  const float* row = scores + (int64_t)r * stride;
  // each thread owns 16 consecutive keys of the chunk; their loads go out first
  constexpr int kPer = kChunk / 256;
  const int64_t s0 = c0 + (int64_t)tid * kPer;
  uint32_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t s = s0 + i;
    keys[i] = s < n ? order_key(row[s]) : 0u;
  }
  // the threshold bin b* of the row, from its histogram (every workgroup of the row
  // finds the same one; the first also records it, and the count of keys above it,
  // for the resolve launch)
  for (int i = tid; i < kHistBins; i += 256) hb[i] = g[i];
  __syncthreads();
  uint32_t bstar, above;
  threshold_bin(hb, k, hpart, &bstar, &above);
  if (blockIdx.y == 0 && tid == 0) {
    meta[2] = bstar;
    meta[3] = above;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += (s0 + i < n && (keys[i] >> 20) >= bstar) ? 1u : 0u;
  // block-wide exclusive prefix of the per-thread counts, one reservation per block
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t incl = mine;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  uint32_t before = incl - mine, total = 0;
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? part[w] : 0u;
    total += part[w];
  }
  if (tid == 0) base_s = total ? atomicAdd(&meta[0], total) : 0u;
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

// Exclusive prefix sum over the block (1024 threads) and the block total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - v, tot = 0;
  for (int w = 0; w < kResolveThreads / 64; ++w) {
    before += w < wave ? wsum[w] : 0u;
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return before;
}

// Digit d (0..1023) of a 1024-bin histogram (one bin per thread) holding the
// need-th largest key, and the count of keys in higher digits.
__device__ __forceinline__ void select_digit(uint32_t c, uint32_t need, uint32_t* wsum, uint32_t* sel) {
  // suffix sum: count of keys in digits >= mine = total - (exclusive prefix)
  uint32_t total;
  const uint32_t before = block_excl_scan(c, wsum, &total);
  const uint32_t ge = total - before, gt = ge - c;
  if (gt < need && ge >= need) {
    sel[0] = threadIdx.x;
    sel[1] = gt;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kResolveThreads) topk_resolve_kernel(const float* scores, int64_t stride,
                                                                       RowPos pos, int m, int k,
                                                                       const uint32_t* state,
                                                                       const uint32_t* cand_key,
                                                                       const uint32_t* cand_idx, uint32_t* bm_ws,
                                                                       int32_t* out_idx, int32_t* out_cnt,
                                                                       float* out_score) {
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t wsum[kResolveThreads / 64];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t bm_lds[2 * kBitmapLdsWords];
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
  const uint32_t* meta = state + (int64_t)r * kRowWords + kHistBins;
  const uint32_t nc = meta[0], bstar = meta[2], above = meta[3];
  const uint32_t* gk = cand_key + (int64_t)r * stride;
  const uint32_t* gi = cand_idx + (int64_t)r * stride;
  // the first kRegCand * kResolveThreads candidates stay in registers for all three passes over them
  uint32_t rk[kRegCand], ri[kRegCand];
#pragma unroll
  for (int j = 0; j < kRegCand; ++j) {
    const uint32_t i = tid + j * kResolveThreads;
    rk[j] = i < nc ? gk[i] : 0u;
    ri[j] = i < nc ? gi[i] : 0u;
  }
  // two 10-bit radix passes over the candidates in bin b*: T and the count to take equal to T
  uint32_t need = (uint32_t)k - above, prefix = bstar;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRegCand; ++j)
      if (tid + j * kResolveThreads < nc && (rk[j] >> (shift + 10)) == prefix)
        atomicAdd(&hist[(rk[j] >> shift) & 1023u], 1u);
    for (uint32_t i = tid + kRegCand * kResolveThreads; i < nc; i += blockDim.x) {
      const uint32_t key = gk[i];
      if ((key >> (shift + 10)) == prefix) atomicAdd(&hist[(key >> shift) & 1023u], 1u);
    }
    __syncthreads();
    select_digit(hist[tid], need, wsum, sel);
    prefix = (prefix << 10) | sel[0];
    need -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix, need_eq = need;           // keep every key > T and the need_eq lowest indices == T
  // bitmaps of the row's indices: kept (keys > T, then the chosen ties) and equal to T
  const int64_t words = (n + 31) / 32;
  uint32_t* bm = words <= kBitmapLdsWords ? bm_lds : bm_ws + (int64_t)r * 2 * ((stride + 31) / 32);
  uint32_t* keep = bm;
  uint32_t* eq = bm + words;
  for (int64_t i = tid; i < 2 * words; i += blockDim.x) bm[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRegCand; ++j)
    if (tid + j * kResolveThreads < nc && rk[j] >= T)
      atomicOr(rk[j] > T ? &keep[ri[j] >> 5] : &eq[ri[j] >> 5], 1u << (ri[j] & 31));
  for (uint32_t i = tid + kRegCand * kResolveThreads; i < nc; i += blockDim.x) {
    const uint32_t key = gk[i];
    if (key >= T) {
      const uint32_t id = gi[i];
      atomicOr(key > T ? &keep[id >> 5] : &eq[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  // each thread owns a contiguous run of bitmap words; ties taken in index order
  const int64_t per = (words + kResolveThreads - 1) / kResolveThreads;
  const int64_t w0 = (int64_t)tid * per, w1 = w0 + per < words ? w0 + per : words;
  uint32_t cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(eq[w]);
  uint32_t tot;
  uint32_t rank = block_excl_scan(cnt, wsum, &tot);
  for (int64_t w = w0; w < w1 && rank < need_eq; ++w) {
    uint32_t e = eq[w];
    while (e && rank < need_eq) {
      const uint32_t b = e & (0u - e);
      keep[w] |= b;
      e ^= b;
      ++rank;
    }
  }
  __syncthreads();
  cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(keep[w]);
  uint32_t o = block_excl_scan(cnt, wsum, &tot);
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t e = keep[w];
    while (e) {
      const int b = __ffs(e) - 1;
      const uint32_t id = (uint32_t)(w * 32 + b);
      if (o < (uint32_t)k) {
        oi[o] = (int32_t)id;
        if (os) os[o] = row[id];
      }
      ++o;
      e &= e - 1;
    }
  }
  if (tid == 0) out_cnt[r] = k;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_index_scores(const CacheView& cv, const ca_index_params& p, const void* qI, const float* w,
                               RowPos pos, int seq_fixed, int n_rows, int64_t max_pos, float* scores,
                               int64_t stride, void* ws_long, hipStream_t st, bool state_zeroed) {
  if (n_rows == 0) return hipSuccess;
  const int64_t max_ne = max_pos / p.ratio;
  const bool long_rows = ws_long != nullptr && topk_use_long(stride, p.k);
  uint32_t* state = long_rows ? (uint32_t*)ws_long : nullptr;   // per-row histograms and counters
  const bool mfma = max_ne > 0 && (cv.fmt == CA_E4M3 || cv.fmt == CA_FP4) && p.n_heads == 8 && p.dim == 64 &&
                   cv.page_shift >= 4;
  if (long_rows && !state_zeroed) {   // cleared before the scoring launch, which may add to the histograms
    const int64_t nz = (int64_t)n_rows * kRowWords;
    hipLaunchKernelGGL(topk_zero_kernel, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st, state, nz);
  }
  if (max_ne == 0) return hipGetLastError();   // no entries yet: nothing to score
  hipEvent_t ev0, ev1;
  timer_events(CA_TIMED_INDEX_SCORES, st, &ev0, &ev1);
  bool hist_done = false;   // the one-row-per-workgroup MFMA kernel makes the histogram itself
  if (mfma) {
    const int64_t chunks = (max_ne + kScoreChunk - 1) / kScoreChunk;
    const bool fp4 = cv.fmt == CA_FP4, qfp4 = p.q_quant == CA_FP4;
    if (seq_fixed >= 0) {
      dim3 grid((unsigned)((n_rows + 3) / 4), (unsigned)chunks);
      if (qfp4)
        CA_LAUNCH((index_scores_fp4_kernel<4>), grid, dim3(256), 0, st, ev0, ev1, cv, p.ratio, p.q_format, qI, w, pos,
                  seq_fixed, n_rows, scores, stride, nullptr, 0, 0);
      else if (fp4)
        CA_LAUNCH((index_scores_fp8_kernel<4, CA_FP4>), grid, dim3(256), 0, st, ev0, ev1, cv, p.ratio, p.q_format, qI,
                  w, pos, seq_fixed, n_rows, scores, stride, nullptr, 0, 0);
      else
        CA_LAUNCH((index_scores_fp8_kernel<4, CA_E4M3>), grid, dim3(256), 0, st, ev0, ev1, cv, p.ratio, p.q_format,
                  qI, w, pos, seq_fixed, n_rows, scores, stride, nullptr, 0, 0);
    } else {
      dim3 grid((unsigned)n_rows, (unsigned)chunks);
      const size_t lds = state != nullptr ? kHistBins * sizeof(uint32_t) : 0;
      if (qfp4)
        CA_LAUNCH((index_scores_fp4_kernel<1>), grid, dim3(256), lds, st, ev0, ev1, cv, p.ratio, p.q_format, qI, w,
                  pos, seq_fixed, n_rows, scores, stride, state, kRowWords, p.k);
      else if (fp4)
        CA_LAUNCH((index_scores_fp8_kernel<1, CA_FP4>), grid, dim3(256), lds, st, ev0, ev1, cv, p.ratio, p.q_format,
                  qI, w, pos, seq_fixed, n_rows, scores, stride, state, kRowWords, p.k);
      else
        CA_LAUNCH((index_scores_fp8_kernel<1, CA_E4M3>), grid, dim3(256), lds, st, ev0, ev1, cv, p.ratio, p.q_format,
                  qI, w, pos, seq_fixed, n_rows, scores, stride, state, kRowWords, p.k);
      hist_done = true;
    }
  } else {
    dim3 grid((unsigned)n_rows, (unsigned)((max_ne + 255) / 256));
    size_t sm = sizeof(float) * p.n_heads * p.dim;
    CA_LAUNCH(index_scores_generic_kernel, grid, dim3(256), sm, st, ev0, ev1, cv, p.n_heads, p.dim, p.ratio,
              p.q_format, qI, w, pos, seq_fixed, scores, stride, p.q_quant == CA_FP4 ? 1 : 0);
  }
  if (state != nullptr && !hist_done) {  // histogram of the scores for the long top-k
    const unsigned chunks = (unsigned)((stride + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(n_rows, chunks), dim3(256), 0, st, scores, stride, pos, p.ratio, p.k,
                       state);
  }
  return hipGetLastError();
}

// [rows][kHistBins + kMetaWords] histogram and counters, candidate keys and
// indices [rows][stride] each, and [rows][2][stride/32] bitmaps for rows too long
// for the LDS bitmaps.
size_t topk_long_workspace(int n_rows, int64_t stride) {
  const size_t words = (size_t)(stride + 31) / 32;
  return (size_t)n_rows * kRowWords * 4 + 2 * (size_t)n_rows * stride * 4 +
         2 * (size_t)n_rows * words * 4 + 256;
}

bool topk_use_long(int64_t stride, int k) { return stride > kTopkLdsKeys && k <= kSortMax; }

hipError_t launch_topk(const float* scores, int64_t stride, RowPos pos, int m, int k, int n_rows,
                       int32_t* out_idx, int32_t* out_cnt, float* out_score, void* ws_long, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  if (ws_long != nullptr && topk_use_long(stride, k)) {
    uint32_t* state = (uint32_t*)ws_long;
    uint32_t* cand_key = state + (int64_t)n_rows * kRowWords;
    uint32_t* cand_idx = cand_key + (int64_t)n_rows * stride;
    uint32_t* bm = cand_idx + (int64_t)n_rows * stride;
    // the histogram was made by the scoring launch (see launch_index_scores); the
    // gather workgroups find the threshold bin from it themselves
    const unsigned chunks = (unsigned)((stride + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(topk_gather_kernel, dim3(n_rows, chunks), dim3(256), 0, st, scores, stride, pos, m, k, state,
                       cand_key, cand_idx);
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(n_rows), dim3(kResolveThreads), 0, st, scores, stride, pos, m, k,
                       state, cand_key, cand_idx, bm, out_idx, out_cnt, out_score);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_rows_kernel, dim3(n_rows), dim3(kTopkThreads), 0, st, scores, stride,
                     pos, m, k, out_idx, out_cnt, out_score);
  return hipGetLastError();
}

}  // namespace ca
