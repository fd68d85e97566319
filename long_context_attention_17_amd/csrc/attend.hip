// Core attention of CSA (gathered top-k entries) and HCA (all eligible
// entries), each followed by the sliding window, in one softmax with a
// learned sink; queries RMSNorm-ed and rotated in the prologue, outputs
// de-rotated in the epilogue.
//
// dsv4 book Ch.6 "Shared key-value MQA"; Ch.7 "Dense attention over heavily
// compressed history", "The 128-token uncompressed sliding window", "Query and
// KV RMSNorm", "Partial RoPE and output de-rotation", "Learned attention
// sinks"; Ch.2 "What an attention head computes" (1/sqrt(c) logit scale).
//
// A query row reads an ordered list of "items": its compressed entries
// (idx[r, 0..cnt) for CSA, 0..floor(t/m')-1 for HCA) followed by its window
// tokens max(0, t-n_win+1)..t.  Decode splits the list into fixed chunks of
// kDecodeSplitItems items (a function of the sequence alone, so a sequence's
// result does not depend on the batch it is in) and a combine kernel merges the
// partial (m, l, o) in split order.
//
// MFMA path (D = 512, bf16 queries, bf16 or fp8-mixed entries, bf16 window):
//   one workgroup = one query row x 64 heads (4 wavefronts x 16 heads).
//   Entry tiles of 32 items are staged in LDS as bf16 (fp8 codes dequantized
//   exactly with the per-tile power-of-two scale during staging), double
//   buffered, the next tile's global loads in flight during the current
//   tile's math.  Because every item is both key and value, the same LDS tile
//   feeds both contractions:
//     S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = the
//                   wavefront's 16 normalized query heads held in registers)
//     O  += P V    (A = P straight from the S^T accumulators: lane l holds head
//                   l%16 and items {4g..4g+3, 16+4g..16+4g+3}, g = l/16, which
//                   is a valid k-slot order as long as V uses the same order;
//                   B = V read with ds_read_b64_tr_b16, the gfx950 LDS
//                   transpose load, from the row-major tile)
//   so P never leaves registers and no transposed copy of the tile is kept.
// Generic path (any D multiple of 64 up to 512, fp32 math): one wavefront
//   per (row, head), items streamed from global memory; used for fp32 caches.
#include "common.h"
#include "kernels.h"

namespace ca {

struct RowInfo {
  int t, seq, win_seq, n_c, w0, total;
};

__device__ __forceinline__ RowInfo row_info(const AttendArgs& a, int r) {
  RowInfo ri;
  ri.t = a.pos ? a.pos[r] : r;
  ri.seq = a.seq_fixed >= 0 ? a.seq_fixed : r;
  ri.win_seq = a.seq_fixed >= 0 ? 0 : r;
  int nc;
  if (a.mode == 0) {
    nc = a.cnt[r];
    nc = nc < 0 ? 0 : (nc > a.k ? a.k : nc);
  } else {
    nc = ri.t >= 0 ? ri.t / a.ratio : 0;
  }
  ri.n_c = nc;
  ri.w0 = ri.t - a.n_win + 1 > 0 ? ri.t - a.n_win + 1 : 0;
  ri.total = ri.t >= 0 ? nc + (ri.t - ri.w0 + 1) : 0;
  return ri;
}

// Source of item j of a row; nullptr when the item must be skipped.
__device__ __forceinline__ const uint8_t* item_ptr(const AttendArgs& a, const RowInfo& ri, int r, int j,
                                                   bool* is_win) {
  if (j < ri.n_c) {
    *is_win = false;
    int64_t e = a.mode == 0 ? (int64_t)a.idx[(int64_t)r * a.k + j] : (int64_t)j;
    if (a.mode == 0 && (e < 0 || e >= ri.t / a.ratio)) return nullptr;
    return a.kv.entry(ri.seq, e);
  }
  *is_win = true;
  int p = ri.w0 + (j - ri.n_c);
  int64_t esz = a.win_fmt == CA_F32 ? 4 : 2;
  return (const uint8_t*)a.win + ((int64_t)ri.win_seq * a.W + p % a.W) * a.D * esz;
}

// Splits of a row; never more than the workspace holds (a row whose position
// exceeds the caller's max_pos is truncated rather than overrunning it).
__device__ __forceinline__ int n_splits_of(const AttendArgs& a, int total) {
  if (a.split_items <= 0) return 1;
  int n = (total + a.split_items - 1) / a.split_items;
  n = n > 0 ? n : 1;
  return n < a.max_splits ? n : a.max_splits;
}

// ======================================================================== generic
template <int NPL>
__global__ void __launch_bounds__(64) attend_generic_kernel(AttendArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, split = blockIdx.z, lane = threadIdx.x;
  const int D = a.D, R = a.R, C = a.D - a.R;
  const RowInfo ri = row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  if (split >= ns) return;
  int j0 = 0, j1 = ri.total;
  if (a.split_items > 0) {
    j0 = split * a.split_items;
    j1 = j0 + a.split_items < ri.total ? j0 + a.split_items : ri.total;
  }
  float qv[NPL], o[NPL];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int d = lane + 64 * i;
    qv[i] = load_act(a.q, a.q_fmt, ((int64_t)r * a.n_heads + h) * D + d);
    ss += qv[i] * qv[i];
    o[i] = 0.0f;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int d = lane + 64 * i;
    qv[i] *= inv * a.q_gain[d];
    float other = __shfl_xor(qv[i], 1, 64);
    if (d >= C) {
      float s, c;
      rope_sincos((double)ri.t, (d - C) >> 1, R, a.base, &s, &c);
      qv[i] = (d & 1) ? other * s + qv[i] * c : qv[i] * c - other * s;
    }
  }
  float m = -INFINITY, l = 0.0f;
  for (int j = j0; j < j1; ++j) {
    bool is_win;
    const uint8_t* p = item_ptr(a, ri, r, j, &is_win);
    if (p == nullptr) continue;
    const int fmt = is_win ? a.win_fmt : a.kv.fmt;
    float x[NPL];
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      int d = lane + 64 * i;
      if (fmt == CA_F32) {
        x[i] = ((const float*)p)[d];
      } else if (fmt == CA_BF16) {
        x[i] = bf16_bits_to_f32(((const uint16_t*)p)[d]);
      } else {  // CA_FP8MIX
        if (d < C) {
          int e = (int8_t)p[D + R + (d >> 6)];
          x[i] = ldexpf(e4m3x2_to_f32((uint32_t)p[d])[0], e);
        } else {
          x[i] = bf16_bits_to_f32(((const uint16_t*)(p + C))[d - C]);
        }
      }
      dot += qv[i] * x[i];
    }
    dot = wave_sum(dot) * a.scale_log2;
    float mn = fmaxf(m, dot);
    float alpha = exp2f(m - mn), pj = exp2f(dot - mn);
    l = l * alpha + pj;
#pragma unroll
    for (int i = 0; i < NPL; ++i) o[i] = o[i] * alpha + pj * x[i];
    m = mn;
  }
  const int hh = h;
  if (a.split_items > 0) {
    int64_t base = ((int64_t)r * a.max_splits + split) * a.n_heads + hh;
#pragma unroll
    for (int i = 0; i < NPL; ++i) a.part_o[base * D + lane + 64 * i] = o[i];
    if (lane == 0) {
      a.part_ml[2 * base] = m;
      a.part_ml[2 * base + 1] = l;
    }
    return;
  }
  const float sk = a.sink[hh] * kLog2e;
  const float M = fmaxf(m, sk);
  const float den = l * exp2f(m - M) + exp2f(sk - M);
  const float f = exp2f(m - M) / den;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int d = lane + 64 * i;
    float v = o[i] * f;
    float other = __shfl_xor(v, 1, 64);
    if (d >= C) {
      float s, c;
      rope_sincos((double)ri.t, (d - C) >> 1, R, a.base, &s, &c);
      v = (d & 1) ? v * c - other * s : v * c + other * s;  // R_{-t}
    }
    int64_t oi = ((int64_t)r * a.n_heads + hh) * D + d;
    if (a.out_fmt == CA_F32) ((float*)a.out)[oi] = v;
    else ((uint16_t*)a.out)[oi] = f32_to_bf16_bits(v);
  }
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.n_heads + hh] = (M + log2f(den)) / kLog2e;
}

// ======================================================================== combine
__global__ void attend_combine_kernel(AttendArgs a) {
  const int r = blockIdx.x, hh = blockIdx.y, d = threadIdx.x;
  const int D = a.D, C = a.D - a.R;
  const RowInfo ri = row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  const float sk = a.sink[hh] * kLog2e;
  float M = sk;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[2 * (((int64_t)r * a.max_splits + s) * a.n_heads + hh)]);
  float den = exp2f(sk - M), acc = 0.0f;
  for (int s = 0; s < ns; ++s) {
    int64_t base = ((int64_t)r * a.max_splits + s) * a.n_heads + hh;
    float ms = a.part_ml[2 * base], ls = a.part_ml[2 * base + 1];
    float wgt = exp2f(ms - M);
    den += ls * wgt;
    if (d < D) acc += a.part_o[base * D + d] * wgt;
  }
  float v = acc / den;
  float other = __shfl_xor(v, 1, 64);
  if (d >= D) return;
  if (d >= C) {
    float s, c;
    rope_sincos((double)ri.t, (d - C) >> 1, a.R, a.base, &s, &c);
    v = (d & 1) ? v * c - other * s : v * c + other * s;
  }
  int64_t oi = ((int64_t)r * a.n_heads + hh) * D + d;
  if (a.out_fmt == CA_F32) ((float*)a.out)[oi] = v;
  else ((uint16_t*)a.out)[oi] = f32_to_bf16_bits(v);
  if (a.lse && d == 0) a.lse[(int64_t)r * a.n_heads + hh] = (M + log2f(den)) / kLog2e;
}

// ======================================================================== MFMA (D = 512)
constexpr int kD = 512;
constexpr int kR = 64;
constexpr int kTile = 32;               // items per tile
constexpr int kPitch = kD + 8;          // bf16 elements per LDS tile row (16 B pad against bank conflicts)
constexpr int kRawPitch = 1024;         // bytes per raw (fp8 record or bf16 window) staging row
constexpr int kMaxItems = 2176;         // item pointers cached in LDS per workgroup (k + window <= 2048 + 128)

template <int KV_FMT>
struct MfmaShared {
  static constexpr int kStages = KV_FMT == CA_FP8MIX ? 3 : 4;
  // bf16 records: the ring holds bf16 tiles directly.  fp8 records: the ring holds raw
  // bytes and one bf16 tile receives the dequantized copy.
  static constexpr int kRingBytes = KV_FMT == CA_FP8MIX ? kTile * kRawPitch : kTile * kPitch * 2;
  __attribute__((aligned(16))) uint8_t ring[kStages][kRingBytes];
  __attribute__((aligned(16))) __bf16 tile[KV_FMT == CA_FP8MIX ? kTile * kPitch : 8];
  const uint8_t* items[kMaxItems];
  int kind[kStages][kTile];             // 0: skipped item, 1: bf16 row, 2: fp8 record
  float rope_cs[kR];                    // (cos, sin) of t * theta_p, p < R/2
};

// Issue the async (global -> LDS) loads of tile `tile_no` into ring stage `st`.
// Every wave issues exactly 8 load instructions (one per item it owns, items
// wave, wave+4, ...), so outstanding-load counts are the same for all tiles.
template <int KV_FMT>
__device__ __forceinline__ void issue_tile(const AttendArgs& a, const RowInfo& ri, int r, int j0, int j1,
                                           int tile_no, int st, MfmaShared<KV_FMT>& sh, const uint8_t* dummy) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int it = wave + 4 * u;
    const int j = j0 + tile_no * kTile + it;
    // the host guarantees j1 - j0 <= kMaxItems (longer rows are split)
    const uint8_t* p = j < j1 ? sh.items[j - j0] : nullptr;
    const bool is_win = j >= ri.n_c;
    const int kind = p == nullptr ? 0 : ((KV_FMT == CA_FP8MIX && !is_win) ? 2 : 1);
    const uint8_t* src = p == nullptr ? dummy : p;
    uint8_t* dst = KV_FMT == CA_FP8MIX ? sh.ring[st] + it * kRawPitch : sh.ring[st] + it * kPitch * 2;
    if (kind == 2) {
      if (lane < 37) __builtin_amdgcn_global_load_lds(src + 16 * lane, (lds_void*)dst, 16, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(src + 16 * lane, (lds_void*)dst, 16, 0, 0);
    }
    if (lane == 0) sh.kind[st][it] = kind;
  }
}

// Wait until at most 8*ahead of this wave's async loads are still in flight.
__device__ __forceinline__ void wait_loads(int ahead) {
  switch (ahead) {
    case 0: __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 2: __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    default: __asm__ volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
  }
}

// fp8 records: dequantize the raw stage into the bf16 tile (each thread: 8 slots
// of 8 channels; content channels scaled by their tile exponent, rotary and
// window rows copied; skipped items zeroed).
__device__ __forceinline__ void convert_tile(const uint8_t* raw, const int* kind, __bf16* tile) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sid = threadIdx.x + 256 * u;
    const int it = sid >> 6, sl = sid & 63;
    const uint8_t* row = raw + it * kRawPitch;
    __bf16* dst = tile + it * kPitch + 8 * sl;
    const int kd = kind[it];
    u32x4 out = {0u, 0u, 0u, 0u};
    if (kd == 1) {
      out = *(const u32x4*)(row + 16 * sl);
    } else if (kd == 2) {
      if (sl < 56) {            // channels 8*sl .. 8*sl+7 < 448: e4m3 codes
        const u32x2 w = *(const u32x2*)(row + 8 * sl);
        const float sc = ldexpf(1.0f, (int)(int8_t)row[kD + kR + (sl >> 3)]);
        bf16x2 c0 = e4m3x2_to_bf16_scaled<false>(w[0], sc), c1 = e4m3x2_to_bf16_scaled<true>(w[0], sc);
        bf16x2 c2 = e4m3x2_to_bf16_scaled<false>(w[1], sc), c3 = e4m3x2_to_bf16_scaled<true>(w[1], sc);
        out[0] = __builtin_bit_cast(uint32_t, c0);
        out[1] = __builtin_bit_cast(uint32_t, c1);
        out[2] = __builtin_bit_cast(uint32_t, c2);
        out[3] = __builtin_bit_cast(uint32_t, c3);
      } else {                  // rotary channels, bf16
        out = *(const u32x4*)(row + 448 + 16 * (sl - 56));
      }
    }
    *(u32x4*)dst = out;
  }
}

// S^T = K Q^T for one 32-item tile: two 16-item blocks x two halves of the 512-dim
// contraction (four independent accumulator chains).  The K fragments are read one
// step ahead of their MFMAs; sched_barrier keeps the compiler from hoisting all 32
// reads at once.  Output: this lane's 8 scaled log2 logits (head li, items 4g..4g+3
// and 16+4g..16+4g+3; -inf for skipped items) and the per-head tile max.
__device__ __forceinline__ void attend_scores(const __bf16* kt, const int* kind, const bf16x8* qreg,
                                              float scale_log2, int li, int g, float* sv, float& tmax) {
  f32x4 s0a = {0.0f, 0.0f, 0.0f, 0.0f}, s1a = s0a, s0b = s0a, s1b = s0a;
  const __bf16* r0 = kt + li * kPitch + 8 * g;
  const __bf16* r1 = kt + (16 + li) * kPitch + 8 * g;
  bf16x8 k0 = *(const bf16x8*)(r0), k1 = *(const bf16x8*)(r1);
  bf16x8 k2 = *(const bf16x8*)(r0 + 256), k3 = *(const bf16x8*)(r1 + 256);
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    bf16x8 n0, n1, n2, n3;
    if (kb < 7) {
      n0 = *(const bf16x8*)(r0 + 32 * (kb + 1));
      n1 = *(const bf16x8*)(r1 + 32 * (kb + 1));
      n2 = *(const bf16x8*)(r0 + 256 + 32 * (kb + 1));
      n3 = *(const bf16x8*)(r1 + 256 + 32 * (kb + 1));
    }
    s0a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[kb], s0a, 0, 0, 0);
    s1a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[kb], s1a, 0, 0, 0);
    s0b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k2, qreg[kb + 8], s0b, 0, 0, 0);
    s1b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k3, qreg[kb + 8], s1b, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kb < 7) {
      k0 = n0;
      k1 = n1;
      k2 = n2;
      k3 = n3;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sv[v] = kind[4 * g + v] ? (s0a[v] + s0b[v]) * scale_log2 : -INFINITY;
    sv[4 + v] = kind[16 + 4 * g + v] ? (s1a[v] + s1b[v]) * scale_log2 : -INFINITY;
    mx = fmaxf(mx, fmaxf(sv[v], sv[4 + v]));
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  tmax = fmaxf(mx, __shfl_xor(mx, 32, 64));
}

// P = 2^(s - m_run) (bf16 A operand, straight from this lane's logits) and O += P V,
// V^T fragments via LDS transpose loads in the same item order, read one column
// block ahead of their MFMA.
__device__ __forceinline__ void attend_pv(const __bf16* kt, const float* sv, float m_run, float& l_part, int li,
                                          int g, f32x4* oacc) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  bf16x8 pa;
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = m_run == -INFINITY ? 0.0f : exp2f(sv[e] - m_run);
    psum += p;
    pa[e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(p));
  }
  l_part += psum;
  const int vrow = 4 * g + (li >> 2), vcol = 4 * (li & 3);
  const __bf16* vbase = kt + vrow * kPitch + vcol;
  bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase));
  bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase + 16 * kPitch));
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    bf16x4 na, nb;
    if (cb < 31) {
      na = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase + 16 * (cb + 1)));
      nb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase + 16 * kPitch + 16 * (cb + 1)));
    }
    bf16x8 vv;
    vv[0] = va[0]; vv[1] = va[1]; vv[2] = va[2]; vv[3] = va[3];
    vv[4] = vb[0]; vv[5] = vb[1]; vv[6] = vb[2]; vv[7] = vb[3];
    oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vv, oacc[cb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (cb < 31) {
      va = na;
      vb = nb;
    }
  }
}

template <int KV_FMT>
__global__ void __launch_bounds__(256) attend_mfma_kernel(AttendArgs a) {
  typedef MfmaShared<KV_FMT> Sh;
  constexpr int NS = Sh::kStages;
  __shared__ Sh sh;

  const int r = blockIdx.x, hg = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const RowInfo ri = row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  if (split >= ns) return;
  int j0 = 0, j1 = ri.total;
  if (a.split_items > 0) {
    j0 = split * a.split_items;
    j1 = j0 + a.split_items < ri.total ? j0 + a.split_items : ri.total;
  }
  const int ntiles = (j1 - j0 + kTile - 1) / kTile;
  const int head_s = hg * 64 + wave * 16 + li;      // head this lane scores (S^T column)
  constexpr int C = kD - kR;

  // ---- prologue: RoPE table for position t, item source table, first async tiles
  if (tid < kR / 2) {
    float sn, cs;
    rope_sincos((double)ri.t, tid, kR, a.base, &sn, &cs);
    sh.rope_cs[2 * tid] = cs;
    sh.rope_cs[2 * tid + 1] = sn;
  }
  const int n_tab = (j1 - j0) < kMaxItems ? (j1 - j0) : kMaxItems;
  for (int i = tid; i < n_tab; i += 256) {
    bool w;
    sh.items[i] = item_ptr(a, ri, r, j0 + i, &w);
  }
  // a valid, finite row used as the source of loads for skipped items: the window token at t
  const uint8_t* dummy = (const uint8_t*)a.win + ((int64_t)ri.win_seq * a.W + ri.t % a.W) * kD * 2;
  __syncthreads();
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) issue_tile<KV_FMT>(a, ri, r, j0, j1, t, t, sh, dummy);

  // ---- query: RMSNorm with gain, RoPE at t, bf16 B-operand fragments (lane: head li, dims 32kb+8g..+7)
  bf16x8 qreg[16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)r * a.n_heads + head_s) * kD;
    float ss = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      u32x4 w = *(const u32x4*)(qrow + 32 * kb + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xFFFF0000u);
        ss += x0 * x0 + x1 * x1;
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss / (float)kD + a.eps);
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      const int d0 = 32 * kb + 8 * g;
      u32x4 w = *(const u32x4*)(qrow + d0);
      f32x4 g0 = *(const f32x4*)(a.q_gain + d0), g1 = *(const f32x4*)(a.q_gain + d0 + 4);
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= inv * (e < 4 ? g0[e] : g1[e - 4]);
      if (d0 >= C) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int p = (d0 + e - C) >> 1;
          const float c = sh.rope_cs[2 * p], sn = sh.rope_cs[2 * p + 1];
          const float x0 = x[e], x1 = x[e + 1];
          x[e] = x0 * c - x1 * sn;
          x[e + 1] = x0 * sn + x1 * c;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[kb][e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(x[e]));
    }
  }

  f32x4 oacc[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) oacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Softmax reference: m_run is fixed by the first tile with a valid item and moves only
  // when a logit exceeds it by more than kBump (log2 units).  Probabilities relative to
  // it stay <= 2^kBump, far inside fp32/bf16 range, so the hot loop never rescales O
  // (no vector ALU work on the accumulators, which then stay in their registers); the
  // rare move leaves the hot loop, rescales O once and finishes the tile.
  constexpr float kBump = 60.0f;
  float m_run = -INFINITY, l_part = 0.0f;
  float sv[8];
  float tmax = -INFINITY;
  int tile = 0;
  while (tile < ntiles) {
    bool pending = false;
    const __bf16* kt = nullptr;
    for (; tile < ntiles; ++tile) {
      const int st = tile % NS;
      const int ahead = (ntiles - 1 - tile) < (NS - 2) ? (ntiles - 1 - tile) : (NS - 2);
      wait_loads(ahead);
      __syncthreads();                                   // tile `tile` landed for every wave
      if (tile + NS - 1 < ntiles)
        issue_tile<KV_FMT>(a, ri, r, j0, j1, tile + NS - 1, (tile + NS - 1) % NS, sh, dummy);
      if (KV_FMT == CA_FP8MIX) {
        convert_tile(sh.ring[st], sh.kind[st], sh.tile);
        __syncthreads();
        kt = sh.tile;
      } else {
        kt = (const __bf16*)sh.ring[st];
      }
      attend_scores(kt, sh.kind[st], qreg, a.scale_log2, li, g, sv, tmax);
      if (__builtin_expect(__any(tmax > m_run + kBump), 0)) {
        pending = true;
        break;
      }
      attend_pv(kt, sv, m_run, l_part, li, g, oacc);
    }
    if (!pending) break;
    // rare path: move the reference up to this tile's max and rescale O
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new);
    l_part *= alpha;
    m_run = m_new;
    float al[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) al[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) oacc[cb][v] *= al[v];
    attend_pv(kt, sv, m_run, l_part, li, g, oacc);
    ++tile;
  }

  // ---- epilogue
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int head_base = hg * 64 + wave * 16;
  if (a.split_items > 0) {
    int64_t pbase = ((int64_t)r * a.max_splits + split) * a.n_heads;
    if (lane < 16) {
      a.part_ml[2 * (pbase + head_base + lane)] = m_run;
      a.part_ml[2 * (pbase + head_base + lane) + 1] = l_tot;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* dst = a.part_o + (pbase + head_base + 4 * g + v) * kD + li;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) dst[16 * cb] = oacc[cb][v];
    }
    return;
  }
  const float sk_own = a.sink[head_s] * kLog2e;
  const float M_own = fmaxf(m_run, sk_own);
  const float den_own = l_tot * exp2f(m_run - M_own) + exp2f(sk_own - M_own);
  const float f_own = exp2f(m_run - M_own) / den_own;
  if (a.lse && lane < 16) a.lse[(int64_t)r * a.n_heads + head_s] = (M_own + log2f(den_own)) / kLog2e;
  float fv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) fv[v] = __shfl(f_own, 4 * g + v, 64);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t obase = ((int64_t)r * a.n_heads + head_base + 4 * g + v) * kD;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float x = oacc[cb][v] * fv[v];
      if (cb >= 28) {                                  // rotary channels 448..511: rotate by R_{-t}
        float other = __shfl_xor(x, 1, 64);
        const int p = (16 * cb + li - C) >> 1;
        const float c = sh.rope_cs[2 * p], sn = sh.rope_cs[2 * p + 1];
        x = (li & 1) ? x * c - other * sn : x * c + other * sn;
      }
      if (a.out_fmt == CA_F32) ((float*)a.out)[obase + 16 * cb + li] = x;
      else ((uint16_t*)a.out)[obase + 16 * cb + li] = f32_to_bf16_bits(x);
    }
  }
}

// ======================================================================== dispatch
int attend_mfma_max_items() { return kMaxItems; }

bool attend_mfma_supported(const AttendArgs& a) {
  return a.D == kD && a.R == kR && a.n_heads % 64 == 0 && a.q_fmt == CA_BF16 &&
         a.win_fmt == CA_BF16 && (a.kv.fmt == CA_BF16 || a.kv.fmt == CA_FP8MIX);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const int splits = a.split_items > 0 ? a.max_splits : 1;
  if (attend_mfma_supported(a)) {
    dim3 grid(a.n_rows, a.n_heads / 64, splits);
    if (a.kv.fmt == CA_FP8MIX)
      hipLaunchKernelGGL(attend_mfma_kernel<CA_FP8MIX>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attend_mfma_kernel<CA_BF16>, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid(a.n_rows, a.n_heads, splits);
    switch (a.D / 64) {
      case 1: hipLaunchKernelGGL(attend_generic_kernel<1>, grid, dim3(64), 0, st, a); break;
      case 2: hipLaunchKernelGGL(attend_generic_kernel<2>, grid, dim3(64), 0, st, a); break;
      case 4: hipLaunchKernelGGL(attend_generic_kernel<4>, grid, dim3(64), 0, st, a); break;
      case 8: hipLaunchKernelGGL(attend_generic_kernel<8>, grid, dim3(64), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split_items <= 0) return e;
  int threads = (a.D + 63) / 64 * 64;
  hipLaunchKernelGGL(attend_combine_kernel, dim3(a.n_rows, a.n_heads), dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ca
