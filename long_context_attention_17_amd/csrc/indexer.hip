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
// 32-bit keys (-0 folded onto +0), a radix select (11-, 11- and 10-bit digits for one row in LDS, a 12-bit histogram then two 10-bit passes over the candidates for long rows) finds the k-th
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

// Loads of a group of G MFMA blocks of 32 keys (key = lane % 32 of each), of a
// wavefront whose keys start at wbase: lane i of wpg holds the pool page of the
// wavefront's i-th page (-1: none).  e4m3 pages: lane half h takes the key's code
// bytes [32h, 32h + 32).  FP4 pages: lane half h takes the bytes [16h, 16h + 16)
// (channels 32h .. 32h + 31) and the E8M0 byte of block h.  NT: e4m3 code bytes
// loaded as non-temporal (keys read once per call, as in decode).
// Every lane loads, unconditionally: a lane without a key (past k1, or on a missing
// page) reads the same bytes of `dummy` (at least 64 B of readable device memory)
// and its key is masked by ok.  Unconditional loads let the compiler count them,
// so the waits in the scoring loop are for one block's loads, not for every load in
// flight.
template <int KF, int G, bool NT>
__device__ __forceinline__ void load_key_group(const CacheView& cv, int wpg, int64_t wbase, int64_t k1,
                                               int64_t gbase, int lane, const uint8_t* dummy, KeyGroup<G>& kg) {
  constexpr int cI = 64;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int64_t s = gbase + 32 * u + (lane & 31);
    const int pgv = __shfl(wpg, (int)((s >> cv.page_shift) - (wbase >> cv.page_shift)), 64);
    const int pg = s < k1 ? pgv : -1;
    kg.ok[u] = pg >= 0;
    const uint8_t* base = cv.pool + (int64_t)(kg.ok[u] ? pg : 0) * cv.page_bytes;
    const int slot = kg.ok[u] ? cv.slot_of(s) : 0;
    if constexpr (KF == CA_FP4) {
      const uint8_t* kp = kg.ok[u] ? base + slot * (cI / 2) + 16 * (lane >> 5) : dummy + 16 * (lane >> 5);
      const uint8_t* sp = kg.ok[u] ? base + ((cI / 2) << cv.page_shift) + slot * (cI / 32) + (lane >> 5) : dummy;
      kg.v0[u] = *(const i32x4*)kp;
      kg.sc[u] = *sp;
    } else {
      const i32x4* kp = (const i32x4*)(kg.ok[u] ? base + slot * cI + 32 * (lane >> 5) : dummy + 32 * (lane >> 5));
      const float* sp = kg.ok[u] ? (const float*)(base + (cI << cv.page_shift)) + slot : (const float*)dummy;
      kg.v0[u] = NT ? __builtin_nontemporal_load(kp) : kp[0];
      kg.v1[u] = NT ? __builtin_nontemporal_load(kp + 1) : kp[1];
      kg.ks[u] = *sp;
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
// A chunk's LDS histogram hb[4096] (complete: after a barrier) into the row's state g:
// the nonzero fine bins, and the 64 coarse bins (fine bins 64c .. 64c + 63 summed) that
// follow the state's 4 counters.  256 threads; integer adds, so order free.
// 256 threads.  Fine bins: thread t adds bins t, t + 256, ... (a wavefront's atomics
// cover 64 consecutive bins each).  Coarse bins: thread t sums the fine bins
// 16t .. 16t + 15 (four 16-byte LDS reads; hb 16-byte aligned), which lie in coarse
// bin t / 4, and the four threads of a coarse bin add their sums with two lane swaps.
__device__ __forceinline__ void add_row_histogram(const uint32_t* hb, uint32_t* g) {
  const int t = threadIdx.x;
  for (int i = t; i < 4096; i += 256) {
    const uint32_t c = hb[i];
    if (c) atomicAdd(&g[i], c);
  }
  const u32x4* src = (const u32x4*)hb + 4 * t;
  u32x4 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = src[i];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) sum += (c[i][0] + c[i][1]) + (c[i][2] + c[i][3]);
  sum += __shfl_xor(sum, 1, 64);
  sum += __shfl_xor(sum, 2, 64);
  if ((t & 3) == 0 && sum) atomicAdd(&g[4096 + 4 + (t >> 2)], sum);
}

// Workgroup barrier ordering LDS only: global loads in flight stay in flight
// (__syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kIdxWaitVm0 = 0x0F70;     // s_waitcnt immediate: vmcnt(0), other counters unconstrained

template <int QPW, int KF, int QF>
__device__ __forceinline__ void index_scores_mfma(CacheView cv, int m, int q_fmt, const void* qI, const float* w,
                                                  RowPos pos, int seq_fixed, int n_rows, float* scores,
                                                  int64_t stride, uint32_t* hist, int hist_words, int hist_k) {
  static_assert(QF == CA_E4M3 || (QF == CA_FP4 && KF == CA_FP4), "FP4 queries meet FP4 keys");
  constexpr int nI = 8, cI = 64;
  constexpr int kQBytes = QF == CA_FP4 ? cI / 2 : cI;              // code bytes per query-head row
  extern __shared__ __attribute__((aligned(16))) uint32_t hs[];
  __shared__ __attribute__((aligned(16))) uint8_t qcodes[32 * cI];  // A operand rows: (query, head)
  __shared__ uint8_t qsc[32][2];                                    // FP4 queries: E8M0 byte per block
  __shared__ float wq[32];                                          // w (* query scale for e4m3) per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * QPW;

  const int seq = seq_fixed >= 0 ? seq_fixed : r0;     // decode: one row per group, row == sequence
  const int64_t k0 = (int64_t)blockIdx.y * kScoreChunk;

  // The prologue's loads go out together, each from an in-range address, and only
  // then are they used: the rows' pos words (first: the first to be waited for), the
  // pool pages of the wavefront's 1,024 keys (lane i: page i; at most 64 as
  // page_shift >= 4; validity applied when used), the query rows and their head
  // weights (rows past the group's queries read row r0 and are zeroed).  All of them
  // are older than the key loads, so waiting for them never waits for a key group
  // (loads complete in order).
  int praw[QPW];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq)
    praw[qq] = pos.pos != nullptr ? pos.pos[r0 + qq < n_rows ? r0 + qq : r0] : 0;
  const int64_t wbase = k0 + (kScoreChunk / 4) * wave;
  const int n_wpg = ((kScoreChunk / 4) >> cv.page_shift) > 0 ? ((kScoreChunk / 4) >> cv.page_shift) : 1;
  const int64_t pi = (wbase >> cv.page_shift) + (lane < n_wpg ? lane : 0);
  const bool pi_ok = lane < n_wpg && pi < cv.max_pages;
  const int praw_pg = cv.max_pages > 0 ? cv.page_table[(int64_t)seq * cv.max_pages + (pi_ok ? pi : 0)] : -1;
  constexpr int kRowsPerWave = 32 / 4;                 // query-head rows (query, head) of each wave
  uint32_t qraw[kRowsPerWave];                         // as loaded: bf16 bits or fp32 bits
  float wraw[kRowsPerWave];                            // the rows' head weights
  const bool q_bf16 = q_fmt == CA_BF16;
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int row = wave + 4 * j, qq = row / nI, h = row % nI, r = r0 + qq;
    const bool ok = qq < QPW && r < n_rows;
    const int64_t i = ((int64_t)(ok ? r : r0) * nI + h) * cI + lane;
    qraw[j] = q_bf16 ? (uint32_t)((const uint16_t*)qI)[i] : ((const uint32_t*)qI)[i];
    wraw[j] = w[(int64_t)(ok ? r : r0) * nI + h];
  }

  int64_t ne[QPW];
  int64_t ne_max = 0;
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    int r = r0 + qq;
    int t = r < n_rows ? pos.of(r, praw[qq]) : 0;
    ne[qq] = r < n_rows ? (t / m < stride ? t / m : stride) : 0;
    ne_max = ne[qq] > ne_max ? ne[qq] : ne_max;
  }
  const int wpg = pi_ok && praw_pg < cv.n_pages ? praw_pg : -1;
  if (k0 >= ne_max) return;                            // uniform over the block
  const bool want_hist = QPW == 1 && hist != nullptr && ne[0] > hist_k;   // uniform
  if (want_hist)
    for (int i = threadIdx.x; i < kHistBins; i += 256) hs[i] = 0u;
  const int64_t k1 = (k0 + kScoreChunk < ne_max) ? k0 + kScoreChunk : ne_max;

  // one-row (decode) workgroups: the wavefront's first two key groups go out before
  // the query rows are prepared (with four rows the registers do not allow it), and
  // the keys, read once, are loaded as non-temporal (prefill row groups re-read them)
  constexpr int G = group_blocks<KF>();
  constexpr int kGroupKeys = 32 * G;
  constexpr int kGroups = kScoreChunk / 4 / kGroupKeys;  // groups per wave
  static_assert(kGroups >= 2, "two key groups in flight");
  constexpr bool kEarly = QPW == 1;
  // the source of lanes without a key: the first 64 B of the query rows (a row holds
  // nI * cI = 512 elements of at least 2 B), always readable
  const uint8_t* kdummy = (const uint8_t*)qI;
  KeyGroup<G> cur, nxt;
  if constexpr (kEarly) {
    // every prologue load has arrived (the query words land with the page ids the key
    // loads need): waited for here, as a builtin the compiler sees, no wait on them is
    // left for after the key loads, where it would be a wait for the key groups too
    // (loads complete in order)
    __builtin_amdgcn_s_waitcnt(kIdxWaitVm0);
    load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, wbase, lane, kdummy, cur);
    load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, wbase + kGroupKeys, lane, kdummy, nxt);
  }

  // prologue: QPW*8 query-head rows quantized to e4m3
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int row = wave + 4 * j, qq = row / nI, r = r0 + qq;
    if (qq < QPW && r < n_rows) {                      // (uniform) rows past the group's queries stay zero
      const float v = __uint_as_float(q_bf16 ? qraw[j] << 16 : qraw[j]);
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
        if (lane == 0) wq[row] = wraw[j];
      } else {
        const int e = pow2_exponent(wave_max(fabsf(v)));
        qcodes[row * cI + lane] = (uint8_t)e4m3_encode(ldexpf(v, -e));
        if (lane == 0) wq[row] = wraw[j] * ldexpf(1.0f, e);
      }
    } else {
      if (lane < kQBytes) qcodes[row * kQBytes + lane] = 0;
      if (lane < 2) qsc[row][lane] = 127;
      if (lane == 0) wq[row] = 0.0f;
    }
  }
  lds_barrier();   // the query rows, their weights and the cleared histogram (LDS only)

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

  // scores of one key group held in kg (keys gbase ..): block u + 1's MFMA is issued
  // before block u's results are read (two accumulators), so the matrix unit's latency
  // overlaps the ReLU, weighting and stores
  auto block_mfma = [&](const KeyGroup<G>& kg, int u) {
    const i32x8 bop = __builtin_shufflevector(kg.v0[u], kg.v1[u], 0, 1, 2, 3, 4, 5, 6, 7);
    const f32x16 z = {};
    if constexpr (QF == CA_FP4)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, z, 4, 4, 0, a_scale, 0, kg.sc[u]);
    else if constexpr (KF == CA_FP4)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, z, 0, 4, 0, 127, 0, kg.sc[u]);
    else
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, z, 0, 0, 0, 127, 0, 127);
  };
  auto score_group = [&](const KeyGroup<G>& kg, int64_t gbase) {
    f32x16 acc_next = block_mfma(kg, 0);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t s = gbase + 32 * u + (lane & 31);
      const f32x16 acc = acc_next;
      if (u + 1 < G) acc_next = block_mfma(kg, u + 1);
      // acc[v]: row 8*(v/4) + 4*(lane/32) + v%4 = (query v/4, head 4*(lane/32) + v%4), key lane%32
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float part = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) part += wl[qq][v] * fmaxf(acc[4 * qq + v], 0.0f);
        // the two lane halves' heads: lanes l and l + 32 both get part(l % 32) + part(l % 32 + 32)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (lane < 32 && s < ne[qq]) {
          const float sc = kg.ok[u] ? (KF == CA_FP4 ? part : part * kg.ks[u]) : -INFINITY;
          scores[(int64_t)(r0 + qq) * stride + s] = sc;
          if (want_hist) atomicAdd(&hs[order_key(sc) >> 20], 1u);
        }
      }
    }
  };
  if constexpr (kEarly) {
    // Decode: two groups in flight (the first two already issued), taken in turn by the
    // two register buffers (no copy between them, which would wait for the loads in
    // flight).
    static_assert(kGroups % 2 == 0, "key groups go in pairs");
    for (int grp = 0; grp < kGroups; grp += 2) {
      const int64_t g0 = wbase + kGroupKeys * grp, g1 = g0 + kGroupKeys;
      if (g0 >= k1) break;
      score_group(cur, g0);
      if (grp + 2 < kGroups) load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, g1 + kGroupKeys, lane, kdummy, cur);
      if (g1 >= k1) break;
      score_group(nxt, g1);
      if (grp + 3 < kGroups) load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, g1 + 2 * kGroupKeys, lane, kdummy, nxt);
    }
  } else {
    // Prefill row groups (four query rows): one group ahead; two buffers taken in turn
    // need more registers than two wavefronts per SIMD leave
    load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, wbase, lane, kdummy, cur);
    for (int grp = 0; grp < kGroups; ++grp) {
      const int64_t gbase = wbase + kGroupKeys * grp;
      if (gbase >= k1) break;
      if (grp + 1 < kGroups) load_key_group<KF, G, kEarly>(cv, wpg, wbase, k1, gbase + kGroupKeys, lane, kdummy, nxt);
      score_group(cur, gbase);
      cur = nxt;
    }
  }
  if (want_hist) {   // the chunk's nonzero bins into the row's histogram (integer adds: order free)
    __syncthreads();
    uint32_t* g = hist + (int64_t)r0 * hist_words;
    add_row_histogram(hs, g);
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
constexpr int kTopkBins = 2048;         // radix digits of 11, 11 and 10 bits

struct TopkShared {
  uint32_t keys[kTopkLdsKeys];
  __attribute__((aligned(16))) uint32_t hist[kTopkBins];
  uint32_t wsum[kTopkThreads / 64];
  uint32_t wsum2[kTopkThreads / 64];
  uint32_t sel_digit, sel_krem;
};

__device__ __forceinline__ uint32_t get_key(const TopkShared& sh, bool in_lds, const float* row, int64_t s) {
  return in_lds ? sh.keys[s] : order_key(row[s]);
}

// The score of an order key (order_key's inverse; -0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

// Exclusive prefix sum over the block of a 64-bit value, and the block total.
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint32_t* wlo, uint32_t* whi, uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) {
    wlo[wave] = (uint32_t)incl;
    whi[wave] = (uint32_t)(incl >> 32);
  }
  __syncthreads();
  uint64_t before = incl - v, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint64_t c = ((uint64_t)whi[i] << 32) | wlo[i];
    before += i < wave ? c : 0;
    tot += c;
  }
  *total = tot;
  return before;
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
  if (in_lds) {
    // 8 keys per thread at a time, all 8 loads issued before the first is stored (slots
    // past n re-read key n - 1); more at once would cost the second workgroup per CU its
    // registers
    constexpr int kBatch = 8;
    for (int64_t b0 = 0; b0 < n; b0 += (int64_t)kBatch * kTopkThreads) {
      float v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t s = b0 + tid + (int64_t)i * kTopkThreads;
        v[i] = row[s < n ? s : n - 1];
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t s = b0 + tid + (int64_t)i * kTopkThreads;
        if (s < n) sh.keys[s] = order_key(v[i]);
      }
    }
  }

  // three radix passes over the keys, on bits 31..21, 20..10 and 9..0
  uint32_t prefix = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int width = pass == 2 ? 10 : 11;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + width));
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < kTopkBins; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += blockDim.x) {
      uint32_t key = get_key(sh, in_lds, row, s);
      if ((key & hi_mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L owns digits 32L .. 32L + 31 (eight 16-byte LDS reads); suffix counts from
      // the top digit down; the one lane whose range holds the krem-th key walks it
      const u32x4* hb = (const u32x4*)&sh.hist[32 * tid];
      uint32_t lsum = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 c = hb[q];
        lsum += (c[0] + c[1]) + (c[2] + c[3]);
      }
      uint32_t incl = lsum;  // inclusive suffix sum over lanes >= tid
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(incl, o, 64);
        if (tid + o < 64) incl += v;
      }
      uint32_t cum = incl - lsum;  // keys with digit > 32 * tid + 31
      if (cum < krem && incl >= krem) {
        for (int q = 7; q >= 0; --q) {
          const u32x4 c = hb[q];
          for (int e = 3; e >= 0; --e) {
            const uint32_t nc = cum + c[e];
            if (cum < krem && nc >= krem) {
              sh.sel_digit = 32 * tid + 4 * q + e;
              sh.sel_krem = krem - cum;
            }
            cum = nc;
          }
        }
      }
    }
    __syncthreads();
    prefix |= sh.sel_digit << shift;
    krem = sh.sel_krem;
    __syncthreads();
  }
  // prefix == T (the k-th largest key); krem == how many keys equal to T to keep: every
  // key > T and the krem lowest-indexed keys == T.  Thread tid owns the keys
  // [tid * per, +per) (per a multiple of 4); one block scan of its counts of keys > T
  // and == T gives the kept keys before its run: those > T, and min(krem, those == T).
  const uint32_t T = prefix, need_eq = krem;
  const int64_t per = (n + 4 * kTopkThreads - 1) / (4 * kTopkThreads) * 4;
  const int64_t s0 = tid * per, s1 = s0 + per < n ? s0 + per : n;
  uint32_t n_gt = 0, n_eq = 0;
  if (in_lds) {
    for (int64_t s = s0; s < s1; s += 4) {
      const u32x4 q = *(const u32x4*)&sh.keys[s];   // keys past n are never counted
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        n_gt += (s + e < s1 && q[e] > T) ? 1u : 0u;
        n_eq += (s + e < s1 && q[e] == T) ? 1u : 0u;
      }
    }
  } else {
    for (int64_t s = s0; s < s1; ++s) {
      const uint32_t key = order_key(row[s]);
      n_gt += key > T ? 1u : 0u;
      n_eq += key == T ? 1u : 0u;
    }
  }
  uint64_t tot;
  const uint64_t before = block_excl_scan64(((uint64_t)n_eq << 32) | n_gt, sh.wsum, sh.wsum2, &tot);
  uint32_t eq_seen = (uint32_t)(before >> 32);
  uint32_t o = (uint32_t)before + (eq_seen < need_eq ? eq_seen : need_eq);
  for (int64_t s = s0; s < s1; ++s) {
    const uint32_t key = get_key(sh, in_lds, row, s);
    const bool take = key > T || (key == T && eq_seen < need_eq);
    eq_seen += key == T ? 1u : 0u;
    if (take) {
      if (o < (uint32_t)k) {
        oi[o] = (int32_t)s;
        if (os) os[o] = key_score(key);
      }
      ++o;
    }
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
constexpr int kCoarseBins = 64;       // coarse histogram: the top 6 key bits
constexpr int kRowWords = kHistBins + kMetaWords + kCoarseBins;   // per-row state: histogram, counters, coarse
static_assert(kRowWords == kTopkRowWords, "per-row long top-k state size");
constexpr int kRegCand = 4;            // candidates per resolve thread held in registers
constexpr int kBitmapLdsWords = 16384;  // two LDS bitmaps of rows up to 524,288 keys (larger rows: workspace)

// Words of an index bitmap of n bits, rounded up to a multiple of 4 (16 B).
__host__ __device__ __forceinline__ int64_t bitmap_words(int64_t n) { return ((n + 31) / 32 + 3) & ~(int64_t)3; }

__global__ void topk_zero_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__device__ __forceinline__ int64_t row_len(RowPos pos, int r, int m, int64_t stride) {
  int t = pos(r);
  int64_t n = t / m;
  return n < stride ? n : stride;
}

__global__ void __launch_bounds__(256) topk_hist_kernel(const float* scores, int64_t stride, RowPos pos,
                                                        int m, int k, uint32_t* state) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kHistBins];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  for (int i = tid; i < kHistBins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const float* row = scores + (int64_t)r * stride;
  constexpr int kPer = kChunk / 256;   // every load issued before the first is used
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t s = c0 + tid + 256 * i;
    v[i] = row[s < n ? s : n - 1];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (c0 + tid + 256 * i < n) atomicAdd(&h[order_key(v[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* g = state + (int64_t)r * kRowWords;
  add_row_histogram(h, g);
}

// Wavefront helper: lane l holds the count of bin l (bin 63 the highest keys).  Returns,
// in every lane, the bin holding the need-th largest key (need >= 1, at most the total)
// and the count of keys in the bins above it.
__device__ __forceinline__ void top_bin_of_64(uint32_t c, uint32_t need, uint32_t* bin, uint32_t* above) {
  const int lane = threadIdx.x & 63;
  uint32_t incl = c;                                   // suffix sum: keys in bins >= lane
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += v;
  }
  const uint64_t ge = __ballot(incl >= need);          // bins 0 .. b hold at least `need` keys at or above
  const int b = 63 - __builtin_clzll(ge);
  *bin = (uint32_t)b;
  *above = __shfl(incl - c, b, 64);
}

__global__ void __launch_bounds__(256) topk_gather_kernel(const float* scores, int64_t stride, RowPos pos,
                                                          int m, int k, uint32_t* state, uint32_t* cand_key,
                                                          uint32_t* cand_idx) {
  __shared__ uint32_t part[4];
  __shared__ uint32_t base_s, bstar_s;
  __shared__ uint32_t fine[kHistBins];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t n = row_len(pos, r, m, stride);
  const int64_t c0 = (int64_t)blockIdx.y * kChunk;
  if (n <= k || c0 >= n) return;
  uint32_t* g = state + (int64_t)r * kRowWords;
  uint32_t* meta = g + kHistBins;
  const float* row = scores + (int64_t)r * stride;
  // One round trip for everything the workgroup reads, all loads unconditional: the
  // row's coarse bins (lane l of each wavefront: bin l), its 4,096 fine bins (thread tid:
  // bins tid + 256 j, staged in LDS) and the chunk's scores (thread tid: keys tid + 256 i;
  // slots past n re-read key n - 1 and are never used)
  constexpr int kPer = kChunk / 256;
  const uint32_t cw = meta[kMetaWords + (tid & 63)];
  uint32_t fw[kHistBins / 256];
#pragma unroll
  for (int j = 0; j < kHistBins / 256; ++j) fw[j] = g[tid + 256 * j];
  const int64_t s0 = c0 + tid;
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t s = s0 + 256 * i;
    v[i] = row[s < n ? s : n - 1];
  }
#pragma unroll
  for (int j = 0; j < kHistBins / 256; ++j) fine[tid + 256 * j] = fw[j];
  lds_barrier();
  // the threshold bin b* of the row (every workgroup of the row finds the same one; the
  // first also records it, and the count of keys above it, for the resolve launch):
  // wavefront 0 finds the coarse bin holding the k-th largest key from the 64 coarse
  // bins, then b* among that coarse bin's 64 fine bins
  if (tid < 64) {
    uint32_t cbin, above_c;
    top_bin_of_64(cw, (uint32_t)k, &cbin, &above_c);
    uint32_t fbin, above_f;
    top_bin_of_64(fine[64 * cbin + tid], (uint32_t)k - above_c, &fbin, &above_f);
    if (tid == 0) {
      bstar_s = 64 * cbin + fbin;
      if (blockIdx.y == 0) {
        meta[2] = 64 * cbin + fbin;
        meta[3] = above_c + above_f;
      }
    }
  }
  lds_barrier();
  const uint32_t bstar = bstar_s;
  uint32_t keys[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) keys[i] = order_key(v[i]);
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += (s0 + 256 * i < n && (keys[i] >> 20) >= bstar) ? 1u : 0u;
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
    const int64_t s = s0 + 256 * i;
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
  __shared__ __attribute__((aligned(16))) uint32_t bm_lds[2 * kBitmapLdsWords];
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint32_t* meta = state + (int64_t)r * kRowWords + kHistBins;
  const uint32_t* gk = cand_key + (int64_t)r * stride;
  const uint32_t* gi = cand_idx + (int64_t)r * stride;
  // the first kRegCand * kResolveThreads candidate slots go into registers (kept for all
  // three passes over them) in the same round trip as the row's position and counters:
  // the slots lie inside the row's candidate arrays (stride > kTopkLdsKeys > kRegCand *
  // kResolveThreads), and those at or past the candidate count are masked once it is
  // known (a row that needs no resolve loads them too and leaves them unused)
  static_assert(kRegCand * kResolveThreads <= kTopkLdsKeys, "speculative candidate slots inside the row");
  uint32_t rk[kRegCand], ri[kRegCand];
#pragma unroll
  for (int j = 0; j < kRegCand; ++j) {
    rk[j] = gk[tid + j * kResolveThreads];
    ri[j] = gi[tid + j * kResolveThreads];
  }
  const uint32_t nc = meta[0], bstar = meta[2], above = meta[3];
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
  // bitmaps of the row's indices: kept (keys > T, then the chosen ties) and equal to T,
  // each a multiple of 4 words, read and cleared 16 B at a time; cleared while the
  // loads are in flight (the radix passes' barriers order it before the first use)
  const int64_t words = bitmap_words(n);
  uint32_t* bm = words <= kBitmapLdsWords ? bm_lds : bm_ws + (int64_t)r * 2 * bitmap_words(stride);
  uint32_t* keep = bm;
  uint32_t* eq = bm + words;
  for (int64_t i = tid; i < 2 * words / 4; i += blockDim.x) ((u32x4*)bm)[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kRegCand; ++j)
    if (tid + j * kResolveThreads >= nc) rk[j] = ri[j] = 0u;
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
  // the last pass's bin of T counts the candidates equal to T: when every one of them
  // is kept (the usual case) they go straight into the kept bitmap (uniform)
  const bool all_eq = hist[T & 1023u] == need_eq;
#pragma unroll
  for (int j = 0; j < kRegCand; ++j)
    if (tid + j * kResolveThreads < nc && rk[j] >= T)
      atomicOr(rk[j] > T || all_eq ? &keep[ri[j] >> 5] : &eq[ri[j] >> 5], 1u << (ri[j] & 31));
  for (uint32_t i = tid + kRegCand * kResolveThreads; i < nc; i += blockDim.x) {
    const uint32_t key = gk[i];
    if (key >= T) {
      const uint32_t id = gi[i];
      atomicOr(key > T || all_eq ? &keep[id >> 5] : &eq[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  // each thread owns a contiguous run of bitmap words (a multiple of 4); ties taken in
  // index order
  const int64_t per = (words / 4 + kResolveThreads - 1) / kResolveThreads * 4;
  const int64_t w0 = (int64_t)tid * per, w1 = w0 + per < words ? w0 + per : words;
  auto popc_run = [&](const uint32_t* b) {
    uint32_t c = 0;
    for (int64_t w = w0; w < w1; w += 4) {
      const u32x4 q = *(const u32x4*)&b[w];
      c += __popc(q[0]) + __popc(q[1]) + __popc(q[2]) + __popc(q[3]);
    }
    return c;
  };
  uint32_t cnt, tot;
  if (!all_eq) {
    cnt = popc_run(eq);
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
  }
  cnt = popc_run(keep);
  uint32_t o = block_excl_scan(cnt, wsum, &tot);
  for (int64_t w4 = w0; w4 < w1; w4 += 4) {
    const u32x4 q = *(const u32x4*)&keep[w4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      uint32_t e = q[x];
      while (e) {
        const int b = __ffs(e) - 1;
        const uint32_t id = (uint32_t)((w4 + x) * 32 + b);
        if (o < (uint32_t)k) {
          oi[o] = (int32_t)id;
          if (os) os[o] = row[id];
        }
        ++o;
        e &= e - 1;
      }
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
  const size_t words = (size_t)bitmap_words(stride);
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
