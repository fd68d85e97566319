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
// tokens max(0, t-n_win+1)..t.  Decode splits the list into chunks whose length
// is a function of the row alone (so a sequence's result does not depend on the
// batch it is in), and a combine kernel merges the partial (m, l, o) in split
// order.
//
// MFMA path (D = 512, bf16 queries, bf16 or fp8-mixed entries, bf16 window):
// persistent workgroups of 4 wavefronts, one unit (row, 64 heads, split) at a
// time; the MFMA section below describes the tiling.
// Generic path (any D multiple of 64 up to 512, fp32 math): one wavefront
//   per (row, head), items streamed from global memory; used for fp32 caches.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "qprep.h"

namespace ca {

struct RowInfo {
  int t, seq, win_seq, n_c, w0, total;
};

// A decode row whose position lies outside [0, max_pos] is out of contract: it gets
// no items (so nothing is read for it and its output is zero), position 0, and the
// call's status word receives CA_STATUS_POS_RANGE (unless !report).  pos_r and cnt_r:
// the row's pos[r] and cnt[r] words as loaded (each read only when the call has that array).
__device__ __forceinline__ RowInfo row_info_of(const AttendArgs& a, int r, int pos_r, int cnt_r,
                                               bool report = true) {
  RowInfo ri;
  bool ok = true;
  if (a.pos) {
    ri.t = pos_r;
    ok = ri.t >= 0 && ri.t <= a.max_pos;
    if (!ok) {
      if (report && threadIdx.x == 0) raise_status(a.status, CA_STATUS_POS_RANGE);
      ri.t = 0;
    }
  } else {
    ri.t = a.t0 + r;
  }
  ri.seq = a.seq_fixed >= 0 ? a.seq_fixed : r;
  ri.win_seq = a.seq_fixed >= 0 ? 0 : r;
  int nc;
  if (a.mode == 0) {
    nc = cnt_r;
    nc = nc < 0 ? 0 : (nc > a.k ? a.k : nc);
  } else {
    nc = ri.t / a.ratio;
  }
  ri.n_c = ok ? nc : 0;
  ri.w0 = ri.t - a.n_win + 1 > 0 ? ri.t - a.n_win + 1 : 0;
  ri.total = ok ? ri.n_c + (ri.t - ri.w0 + 1) : 0;
  return ri;
}
__device__ __forceinline__ RowInfo row_info(const AttendArgs& a, int r) {
  return row_info_of(a, r, a.pos != nullptr ? a.pos[r] : 0, a.mode == 0 ? a.cnt[r] : 0);
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

// Split length of a row of `total` items: a function of the row alone (never
// longer than split_cap).
__device__ __forceinline__ int split_len_of(const AttendArgs& a, int total) {
  return split_plan_len32(total, a.split_min, a.split_div, a.split_cap);
}

// Splits of a row.  Rows within the call's max_pos never need more than the
// workspace holds (plan_max_splits); the cap only guards the workspace.
__device__ __forceinline__ int n_splits_of(const AttendArgs& a, int total) {
  if (a.split_min <= 0) return 1;
  const int n = split_plan_count32(total, a.split_min, a.split_div, a.split_cap);
  return n < a.max_splits ? n : a.max_splits;
}

// Item range [j0, j1) of split `split` of a row.
__device__ __forceinline__ void split_range(const AttendArgs& a, int total, int split, int* j0, int* j1) {
  if (a.split_min <= 0) {
    *j0 = 0;
    *j1 = total;
    return;
  }
  const int len = split_len_of(a, total);
  *j0 = split * len;
  *j1 = *j0 + len < total ? *j0 + len : total;
}

// ======================================================================== generic
template <int NPL>
__global__ void __launch_bounds__(64) attend_generic_kernel(AttendArgs a) {
  const int r = blockIdx.x, h = blockIdx.y, split = blockIdx.z, lane = threadIdx.x;
  const int D = a.D, R = a.R, C = a.D - a.R;
  const RowInfo ri = row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  if (split >= ns) return;
  int j0, j1;
  split_range(a, ri.total, split, &j0, &j1);
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
  if (a.split_min > 0) {
    int64_t base = ((int64_t)r * a.max_splits + split) * a.n_heads + hh;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {   // partials no finer than the output
      if (a.part_bf16) ((uint16_t*)a.part_o)[base * D + lane + 64 * i] = f32_to_bf16_bits(o[i]);
      else a.part_o[base * D + lane + 64 * i] = o[i];
    }
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
// Merge of a row's split partials (m, l, o) in split order, with the sink in the
// denominator, then de-rotation of the rotary channels.  A thread owns 4 channels
// of one head (D/4 threads per head, 512 / (D/4) heads per workgroup); the partials
// of up to kCombineUnroll splits are all loaded before any is combined: the loads keep
// the partials' own format (BF: bf16), widened only where they are used, so that no
// load waits for the one before it.
constexpr int kCombineUnroll = 16;

// 4 partial values as loaded: 4 fp32, or (BF) 4 bf16 in two words.
template <bool BF>
using PartRun = typename std::conditional<BF, u32x2, f32x4>::type;
template <bool BF>
__device__ __forceinline__ PartRun<BF> load_part_run(const AttendArgs& a, int64_t e) {
  if constexpr (BF) return *(const u32x2*)((const uint16_t*)a.part_o + e);
  else return *(const f32x4*)(a.part_o + e);
}
template <bool BF>
__device__ __forceinline__ f32x4 widen_part_run(PartRun<BF> w) {
  if constexpr (BF)
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xFFFF0000u)};
  else return w;
}

template <bool BF>
__global__ void __launch_bounds__(512) attend_combine_kernel(AttendArgs a) {
  const int D = a.D, C = a.D - a.R, tph = D / 4;
  const int r = blockIdx.x, hh = blockIdx.y * (512 / tph) + threadIdx.x / tph, d = 4 * (threadIdx.x % tph);
  if (hh >= a.n_heads) return;
  const RowInfo ri = row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  const int64_t base0 = (int64_t)r * a.max_splits * a.n_heads + hh;   // (split s: + s * n_heads)
  const float sk = a.sink[hh] * kLog2e;
  float ms[kCombineUnroll], ls[kCombineUnroll];
  PartRun<BF> os[kCombineUnroll];
#pragma unroll
  for (int s = 0; s < kCombineUnroll; ++s) {          // splits past ns load split ns - 1 again (unused)
    const int64_t b = base0 + (int64_t)(s < ns ? s : ns - 1) * a.n_heads;
    const f32x2 ml = *(const f32x2*)(a.part_ml + 2 * b);
    ms[s] = ml[0];
    ls[s] = ml[1];
    os[s] = load_part_run<BF>(a, b * D + d);
  }
  float M = sk;
#pragma unroll
  for (int s = 0; s < kCombineUnroll; ++s)
    if (s < ns) M = fmaxf(M, ms[s]);
  for (int s = kCombineUnroll; s < ns; ++s) M = fmaxf(M, a.part_ml[2 * (base0 + (int64_t)s * a.n_heads)]);
  float den = exp2f(sk - M);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kCombineUnroll; ++s) {
    if (s < ns) {
      const float w = exp2f(ms[s] - M);
      den += ls[s] * w;
      const f32x4 o = widen_part_run<BF>(os[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += o[e] * w;
    }
  }
  for (int s = kCombineUnroll; s < ns; ++s) {
    const int64_t b = base0 + (int64_t)s * a.n_heads;
    const float w = exp2f(a.part_ml[2 * b] - M);
    den += a.part_ml[2 * b + 1] * w;
    const f32x4 o = widen_part_run<BF>(load_part_run<BF>(a, b * D + d));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e] * w;
  }
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = acc[e] / den;
  if (d >= C) {                                        // rotary pairs (d, d+1), (d+2, d+3): rotate by R_{-t}
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int p = (d + e - C) >> 1;
      double th = 1.0, bp = a.rope_step;
      for (int k = 0; (p >> k) != 0; ++k) {
        th = ((p >> k) & 1) ? th * bp : th;
        bp *= bp;
      }
      const double rev = (double)ri.t * th * 0.15915494309189535;   // 1 / (2 pi)
      const float fr = (float)(rev - floor(rev));
      const float c = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
      const float x0 = v[e], x1 = v[e + 1];
      v[e] = x0 * c + x1 * sn;
      v[e + 1] = x1 * c - x0 * sn;
    }
  }
  const int64_t oi = ((int64_t)r * a.n_heads + hh) * D + d;
  if (a.out_fmt == CA_F32) {
    *(f32x4*)((float*)a.out + oi) = v;
  } else {
    u32x2 w;
    w[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[0], (__bf16)v[1]});
    w[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2], (__bf16)v[3]});
    *(u32x2*)((uint16_t*)a.out + oi) = w;
  }
  if (a.lse && d == 0) a.lse[(int64_t)r * a.n_heads + hh] = (M + log2f(den)) / kLog2e;
}

// The same merge for partials of the MFMA path, which its epilogue writes in the
// accumulator layout: per (row, split, 64-head group) a block
// [pair][half][cb][v/4][lane][v%4] of fp32 (or bf16), element v of `lane` being
// channel 256*half + 32*cb + 8(v/4) + 4(lane/32) + v%4 of head 32*pair + lane%32 of
// the group.  Workgroup = (row, head group, half, cb); thread (pair, v/4, lane)
// reads one run per split (4 channels of one head), so every wavefront load is 1 KB
// (512 B) contiguous.  The per-(split, head) weights exp2(m_s - M) and the
// per-head denominators are formed once per workgroup in LDS (8 threads per head,
// each over every 8th split, reduced in a fixed order), while the first splits'
// partial rows are already in flight.
constexpr int kCombineLdsSplits = 64;   // splits whose weights sit in LDS (more: read from the partials)

template <bool BF>
__global__ void __launch_bounds__(512) attend_combine_acc_kernel(AttendArgs a) {
  constexpr int D = 512, C = D - 64;
  __shared__ float w_s[kCombineLdsSplits][64];         // exp2(m_s - M) per (split, head of the group)
  __shared__ float red[8][64], red2[8][64];            // per (split group, head) partial max / sum
  __shared__ float M_s[64];
  const int r = blockIdx.x, n_hg = a.n_heads >> 6, n_ms = a.max_splits;
  const int hg = blockIdx.y >> 4, half = (blockIdx.y >> 3) & 1, cb = blockIdx.y & 7;
  const int t = threadIdx.x, pair = t >> 8, vq = (t >> 6) & 3, lane = t & 63;
  const int hq = 32 * pair + (lane & 31);               // the thread's head in the group
  const int h = hg * 64 + hq;
  const int c = 256 * half + 32 * cb + 8 * vq + 4 * (lane >> 5);   // first of its 4 channels
  auto o_at = [&](int s) {                             // the thread's run of split s, as loaded
    const int64_t e = (((int64_t)r * n_ms + s) * n_hg + hg) * (64 * D) + (pair * 2 + half) * 8192 +
                      (cb * 4 + vq) * 256 + 4 * lane;
    return load_part_run<BF>(a, e);
  };
  // Every load goes out before anything waits on the row's split count: the row's
  // position and count words, the sinks, this thread's (m, l) pairs (head hh, splits g
  // and g + 8) and the first splits' partial runs, all within the workspace's
  // max_splits; those of splits the row does not have are never used (past max_splits:
  // split max_splits - 1 again).
  const int hh = t & 63, g = t >> 6;
  const int pos_r = a.pos != nullptr ? a.pos[r] : 0, cnt_r = a.mode == 0 ? a.cnt[r] : 0;
  const float sink_h = a.sink[hg * 64 + hh] * kLog2e;
  const float sink_own = a.sink[h] * kLog2e;
  // (m, l) pairs first and unconditionally (splits past max_splits read the last one,
  // never used): the reduction that needs them then waits for them alone, the partial
  // runs behind them staying in flight (loads complete in order)
  const int64_t base = ((int64_t)r * n_ms) * a.n_heads + hg * 64 + hh;
  const f32x2 ml0 = *(const f32x2*)(a.part_ml + 2 * (base + (int64_t)(g < n_ms ? g : n_ms - 1) * a.n_heads));
  const f32x2 ml1 = *(const f32x2*)(a.part_ml + 2 * (base + (int64_t)(g + 8 < n_ms ? g + 8 : n_ms - 1) * a.n_heads));
  PartRun<BF> os[kCombineUnroll];
#pragma unroll
  for (int s = 0; s < kCombineUnroll; ++s) os[s] = o_at(s < n_ms ? s : n_ms - 1);
  const RowInfo ri = row_info_of(a, r, pos_r, cnt_r);
  const int ns = n_splits_of(a, ri.total);

  // per head of the group: M = max(sink, m_s), den = exp2(sink - M) + sum_s l_s exp2(m_s - M),
  // the sums over the splits of each group g (s = g, g + 8, ...) added in split order
  {
    float mx = -INFINITY;
    if (g < ns) mx = ml0[0];
    if (g + 8 < ns) mx = fmaxf(mx, ml1[0]);
    for (int s = g + 16; s < ns; s += 8) mx = fmaxf(mx, a.part_ml[2 * (base + (int64_t)s * a.n_heads)]);
    red[g][hh] = mx;
    __syncthreads();
    float M = sink_h;
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, red[i][hh]);
    float dp = 0.0f;
    if (g < ns) {
      const float w = exp2f(ml0[0] - M);
      dp += ml0[1] * w;
      w_s[g][hh] = w;
    }
    if (g + 8 < ns) {
      const float w = exp2f(ml1[0] - M);
      dp += ml1[1] * w;
      w_s[g + 8][hh] = w;
    }
    for (int s = g + 16; s < ns; s += 8) {
      const float w = exp2f(a.part_ml[2 * (base + (int64_t)s * a.n_heads)] - M);
      dp += a.part_ml[2 * (base + (int64_t)s * a.n_heads) + 1] * w;
      if (s < kCombineLdsSplits) w_s[s][hh] = w;
    }
    red2[g][hh] = dp;
    if (g == 0) M_s[hh] = M;
    __syncthreads();
  }
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const float M = M_s[hq];
  float den = exp2f(sink_own - M);
#pragma unroll
  for (int i = 0; i < 8; ++i) den += red2[i][hq];
  auto weight = [&](int s) {
    if (s < kCombineLdsSplits) return w_s[s][hq];
    return exp2f(a.part_ml[2 * (((int64_t)r * a.max_splits + s) * a.n_heads + h)] - M);
  };
#pragma unroll
  for (int s = 0; s < kCombineUnroll; ++s) {
    if (s < ns) {
      const float w = weight(s);
      const f32x4 o = widen_part_run<BF>(os[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += o[e] * w;
    }
  }
  for (int s = kCombineUnroll; s < ns; ++s) {
    const f32x4 o = widen_part_run<BF>(o_at(s));
    const float w = weight(s);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += o[e] * w;
  }
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = acc[e] / den;
  if (c >= C) {                                        // rotary pairs (c, c + 1), (c + 2, c + 3): rotate by R_{-t}
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int p = (c + e - C) >> 1;
      double th = 1.0, bp = a.rope_step;
      for (int k = 0; (p >> k) != 0; ++k) {
        th = ((p >> k) & 1) ? th * bp : th;
        bp *= bp;
      }
      const double rev = (double)ri.t * th * 0.15915494309189535;   // 1 / (2 pi)
      const float fr = (float)(rev - floor(rev));
      const float co = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
      const float x0 = v[e], x1 = v[e + 1];
      v[e] = x0 * co + x1 * sn;
      v[e + 1] = x1 * co - x0 * sn;
    }
  }
  const int64_t oi = ((int64_t)r * a.n_heads + h) * D + c;
  if (a.out_fmt == CA_F32) {
    *(f32x4*)((float*)a.out + oi) = v;
  } else {
    u32x2 w;
    w[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[0], (__bf16)v[1]});
    w[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2], (__bf16)v[3]});
    *(u32x2*)((uint16_t*)a.out + oi) = w;
  }
  if (a.lse && half == 0 && cb == 0 && vq == 0 && lane < 32) a.lse[(int64_t)r * a.n_heads + h] = (M + log2f(den)) / kLog2e;
}

// ======================================================================== MFMA (D = 512)
// v_mfma_f32_32x32x16_bf16 lane layouts (l = lane, 0..63):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C (32 x 32): element v of lane l is row 8*(v/4) + 4*(l/32) + v%4, column l%32
// Workgroup = one query row x 64 heads = two wavefront pairs; a pair shares 32
// heads.  Ring tiles hold 64 items.  Wavefront `half` of a pair
//   * scores the items 32*half .. +31 of the tile over all 512 channels:
//     S^T = K Q^T, items on the rows, so element v of lane l is the logit of head
//     l%32 for item 8*(v/4) + 4*(l/32) + v%4 (queries stay in registers);
//   * accumulates O^T = V^T P^T for the channels 256*half .. +255 over all 64
//     items, with its own probabilities and its partner's, swapped through LDS as
//     bf16 fragments.  The lane's 16 probabilities are directly the B operand (P^T:
//     column = head l%32) for the k-slot order {items 0-3, 8-11 | 4-7, 12-15} (and
//     +16); V^T is the A operand, fed in the same order with LDS transpose loads
//     (ds_read_b64_tr_b16: a 16-lane group reading a 4-row x 16-column block gets
//     one column per lane).  Element v of lane l of column block cb is then channel
//     32*cb + 8*(v/4) + 4*(l/32) + v%4 of head l%32: a lane holds runs of 4
//     channels of its own head, so the epilogue scales, de-rotates and stores them
//     with no exchange between lanes.
// A pair keeps one softmax reference max; the rare move of it is decided
// workgroup-wide so that its extra exchange can use a barrier.
constexpr int kD = 512;
constexpr int kR = 64;
constexpr int kRows = 64;               // items per ring tile
constexpr int kPitch = kD + 8;          // bf16 elements per LDS tile row (1040 B)
constexpr int kRawPitch = 592;          // bytes per raw fp8 staging row (584 B record, 16 B granules)
constexpr int kMaxItems = 2176;         // items per workgroup (k + window <= 2048 + 128); longer rows are split
constexpr int kWaitVm0 = 0x0F70;        // s_waitcnt immediate: vmcnt(0), other counters unconstrained
constexpr uint32_t kNoItem = 0xFFFFFFFFu;
constexpr uint32_t kWinFlag = 0x80000000u;
constexpr float kNoMax = -1.0e30f;      // running max before any valid item (finite: no inf - inf)

// LDS row of tile item i: within each 16-item block the 4x4 (i%4, i/4) index is
// transposed, so that the 16 rows a quarter-wavefront reads for a K fragment and
// the 4 rows a 16-lane group reads for a V transpose load (items 4a..4a+3) all sit
// in different LDS banks at the 1040 B row pitch.
__device__ __forceinline__ int mx_row(int i) { return (i & ~15) | ((i & 3) << 2) | ((i >> 2) & 3); }

template <int KV_FMT>
struct MxCfg {
  static constexpr bool kFp8 = KV_FMT == CA_FP8MIX;
  // bf16 entries: the ring holds the tiles the MFMAs read.  fp8 entries: the ring
  // holds raw records and one bf16 tile receives the dequantized copy.
  static constexpr int kStages = 2;
  static constexpr int kStageBytes = kFp8 ? kRows * kRawPitch : kRows * kPitch * 2;
  static constexpr int kLoadsPerWave = kRows / 4;       // one row per load instruction
};

// Prefill (one sequence per call) with bf16 entries: the sequence's page-table row is
// copied to LDS once per workgroup (rows of up to kLdsPages pages), so that the units'
// item tables need no global page-table loads.  (fp8 workgroups have no LDS left.)
constexpr int kLdsPages = 2048;

template <int KV_FMT>
struct MxShared {
  typedef MxCfg<KV_FMT> C;
  __attribute__((aligned(16))) uint8_t ring[C::kStages][C::kStageBytes];
  __attribute__((aligned(16))) __bf16 tile[C::kFp8 ? kRows * kPitch : 8];
  __attribute__((aligned(16))) bf16x8 pex[4][64][2];    // probabilities of each wavefront (P^T fragments)
  uint32_t items[kMaxItems];            // item sources: pool record index, or kWinFlag | window row
  int32_t pt[C::kFp8 ? 1 : kLdsPages];  // bf16 prefill: the sequence's page-table row
  uint32_t valid[C::kStages][4];        // bit u of valid[st][w]: ring row w + 4u holds a real item
  float tmx[4][32];                     // per-head tile max of each wavefront
  __attribute__((aligned(16))) int bump[4];   // wavefront wants to move its reference max
  float lsum[4][32];                    // epilogue: per-head probability sums
  float rope_cs[kR];                    // (cos, sin) of t * theta_p, p < R/2
  __attribute__((aligned(16))) float gain[kD];   // query RMSNorm gain x logit scale x log2(e)
};

// Item table of a unit: items j0 .. j0 + n_tab - 1 as item_src reads them, built
// in groups of kTabGroup items per thread, in phases, so that the dependent loads
// of a group overlap (entry indices, CSA: the selected ones; then page-table
// entries; then offsets).  after_issue() runs once, right after the first group's
// last loads are issued (the caller's own loads then queue behind them).
constexpr int kTabGroup = 3;
template <int MODE, class F>
__device__ __forceinline__ void mx_item_table(const AttendArgs& a, const RowInfo& ri, int r, int j0, int n_tab,
                                              uint32_t* items, const int32_t* pt_lds, const F& after_issue) {
  const int tid = threadIdx.x;
  n_tab = __builtin_amdgcn_readfirstlane(n_tab);
  if (n_tab <= 0) after_issue();
  for (int g0 = 0; g0 < n_tab; g0 += 256 * kTabGroup) {
    int32_t e[kTabGroup], pg[kTabGroup];
    // loads are unconditional (from clamped, in-range addresses) inside one
    // workgroup-uniform branch, and kept apart from their uses, so that no wait
    // separates them
#pragma unroll
    for (int k = 0; k < kTabGroup; ++k) {
      const int i = g0 + tid + 256 * k, j = j0 + i;
      e[k] = i < n_tab && j < ri.n_c ? j : -1;
    }
    if (MODE == 0 && a.k > 0) {
      int32_t x[kTabGroup];
#pragma unroll
      for (int k = 0; k < kTabGroup; ++k) x[k] = a.idx[(int64_t)r * a.k + (e[k] >= 0 ? e[k] : 0)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kTabGroup; ++k) e[k] = e[k] >= 0 ? x[k] : -1;
    }
#pragma unroll
    for (int k = 0; k < kTabGroup; ++k) pg[k] = -1;
    if (a.kv.max_pages <= 0 && g0 == 0) after_issue();
    if (a.kv.max_pages > 0) {
      int32_t x[kTabGroup];
      bool ok[kTabGroup];
#pragma unroll
      for (int k = 0; k < kTabGroup; ++k) {
        const int v = e[k], pi = v >> a.kv.page_shift;
        ok[k] = v >= 0 && (MODE != 0 || v < ri.t / a.ratio) && pi < a.kv.max_pages;
        x[k] = pt_lds != nullptr ? pt_lds[ok[k] ? pi : 0]
                                 : a.kv.page_table[(int64_t)ri.seq * a.kv.max_pages + (ok[k] ? pi : 0)];
      }
      __builtin_amdgcn_sched_barrier(0);
      if (g0 == 0) after_issue();
#pragma unroll
      for (int k = 0; k < kTabGroup; ++k) pg[k] = ok[k] ? x[k] : -1;
    }
#pragma unroll
    for (int k = 0; k < kTabGroup; ++k) {
      const int i = g0 + tid + 256 * k, j = j0 + i;
      if (i < n_tab) {
        uint32_t off;
        if (j < ri.n_c) {
          const int32_t p = pg[k];
          off = (p < 0 || p >= a.kv.n_pages)
                    ? kNoItem
                    : (uint32_t)(((int64_t)p << a.kv.page_shift) | a.kv.slot_of(e[k]));
        } else {
          const int w = ri.w0 + (j - ri.n_c);
          off = kWinFlag | (uint32_t)((int64_t)ri.win_seq * a.W + w % a.W);
        }
        items[i] = off;
      }
    }
  }
}

// Source of an item-table entry: record `off` of the pool in page order (page off >> shift,
// slot off & (page size - 1)), or row off & ~kWinFlag of the bf16 window.  The host keeps
// n_pages * page size and the window's rows below 2^31 - 1, so the flag bit and kNoItem
// never collide with a real item.
__device__ __forceinline__ const uint8_t* item_src(const AttendArgs& a, uint32_t off) {
  return (off & kWinFlag) ? (const uint8_t*)a.win + (uint64_t)(off & ~kWinFlag) * (kD * 2)
                          : (const uint8_t*)a.kv.pool + (uint64_t)(off >> a.kv.page_shift) * a.kv.page_bytes +
                                (uint64_t)(off & ((1u << a.kv.page_shift) - 1u)) * a.kv.stride;
}

// One async global -> LDS load of 16 B per lane (lane l: g + 16 l -> LDS d + 16 l),
// with the wavefront-uniform addresses in scalar registers.  Written as asm so that
// the compiler does not treat it as an LDS event of unknown order (which would force
// full drains of the LDS read counter in the MFMA loops).  It writes no register;
// its completion is awaited with explicit vmcnt waits, and a compiler-inserted vmcnt
// wait can only count it as extra, i.e. wait longer.  m0 is restored afterwards.
__device__ __forceinline__ void lds_load16(uint64_t g, uint32_t d) {
  const uint32_t lane16 = 16u * (threadIdx.x & 63u);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(d), "v"(lane16), "s"(g)
      : "memory");
}

// Async (global -> LDS) loads of ring tile `tile_no` into stage `st`, split so
// that the load instructions can be spread between MFMAs.  Row w + 4u belongs to
// wavefront w, which issues exactly kLoadsPerWave instructions per tile, so
// outstanding-load counts are the same for all tiles.  Rows without an item load
// a finite dummy row and are masked.  fp8 stages take the first 592 B of every row
// (a whole record); window rows of an fp8 workgroup reach the bf16 tile through
// mx_convert's own loads (what their ring rows receive is never read).
template <int KV_FMT>
struct MxIssue {
  uint64_t src;       // lane u < kLoadsPerWave: source of row w + 4u
  uint32_t dst;       // LDS address of the ring stage (wavefront-uniform)
  int wave;           // wavefront index (uniform)
  bool on;            // wavefront-uniform: a tile is being loaded

  // Row sources of this wavefront, and its valid bits in sh.valid[st][w].
  template <class SH>
  __device__ __forceinline__ void prepare(const AttendArgs& a, int j0, int j1, int tile_no, int st, SH& sh,
                                          const uint8_t* dummy, bool enable) {
    typedef MxCfg<KV_FMT> C;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    on = enable;
    dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)sh.ring[st]);
    if (!enable) return;
    uint32_t off = kNoItem;
    if (lane < C::kLoadsPerWave) {
      const int j = j0 + tile_no * kRows + wave + 4 * lane;
      // j1 - j0 <= kMaxItems (the kernel caps it), so j - j0 indexes the item table
      off = j < j1 ? sh.items[j - j0] : kNoItem;
    }
    const uint64_t ok = __ballot(off != kNoItem);
    if (lane == 0) sh.valid[st][wave] = (uint32_t)ok;
    src = (uint64_t)(uintptr_t)(off == kNoItem ? dummy : item_src(a, off));
  }

  // (callers test `on` once, outside their instruction stream)
  __device__ __forceinline__ void row(int u) const {
    typedef MxCfg<KV_FMT> C;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)src, u);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(src >> 32), u);
    const int it = wave + 4 * u;
    const uint32_t d = C::kFp8 ? dst + it * kRawPitch : dst + mx_row(it) * (kPitch * 2);
    if (C::kFp8 && (threadIdx.x & 63) >= kRawPitch / 16) return;
    lds_load16(((uint64_t)hi << 32) | lo, d);
  }

  __device__ __forceinline__ void all() const {
    if (!on) return;
#pragma unroll
    for (int u = 0; u < MxCfg<KV_FMT>::kLoadsPerWave; ++u) row(u);
  }
};

// fp8 records: dequantize a raw stage into the bf16 tile; wavefront w handles the
// rows it = 4u + w (u < 16), whose LDS row is mx_row(it) = 16(u/4) + 4w + u%4.
// WIN: the tile reaches the window, whose rows (it >= n_c - jt: bf16 in global
// memory) go straight into their bf16 tile rows as async global -> LDS loads,
// issued first so that their one round trip overlaps the passes over the records
// and awaited (vmcnt(0)) at the end; the passes then skip those rows.
// Passes, each without a branch per row on the common path (a wavefront's LDS
// accesses take effect in program order, so later passes overwrite earlier ones):
//  1. content channels: lanes sl < 56 scale the 8 e4m3 codes of channels 8sl..8sl+7
//     by the tile exponent of their 64-channel tile, in batches of four rows whose
//     LDS reads are all issued before any conversion;
//  2. rotary channels: the 16 rows' 128 B of bf16 copied by all 64 lanes;
//  3. only for tiles with rows without an item: those rows are zeroed (finite V).
template <bool WIN>
__device__ __forceinline__ void mx_convert(const AttendArgs& a, const uint8_t* raw, const uint32_t* valid,
                                           const uint32_t* items, int jt, int j0, int n_c, __bf16* tile) {
  constexpr int CC = kD - kR;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), sl = threadIdx.x & 63;
  const uint32_t vb = __builtin_amdgcn_readfirstlane(valid[wave]) & 0xFFFFu;
  const uint8_t* rw = raw + wave * kRawPitch;            // row u of this wavefront: + 4u * kRawPitch
  __bf16* tw = tile + 4 * wave * kPitch;                 // row u: + (16(u/4) + u%4) * kPitch
  auto trow = [](int u) { return (16 * (u >> 2) + (u & 3)) * kPitch; };
  int u_rec = kRows / 4;                                 // rows u < u_rec hold records (if valid)
  if constexpr (WIN) {
    const int n_rec = n_c - jt;                          // tile rows it < n_rec are records
    u_rec = __builtin_amdgcn_readfirstlane(n_rec <= wave ? 0 : min(kRows / 4, (n_rec - wave + 3) >> 2));
    // lane u < 16: source of row u if it is a window row (else window row 0, never loaded)
    uint32_t off = kWinFlag;
    if (sl < kRows / 4 && sl >= u_rec && ((vb >> sl) & 1u)) off = items[jt + 4 * sl + wave - j0];
    const uint64_t src = (uint64_t)(uintptr_t)item_src(a, off);
    typedef __attribute__((address_space(3))) __bf16 lds_bf16;
    const uint32_t tb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_bf16*)tw);
#pragma unroll 1
    for (int u = u_rec; u < kRows / 4; ++u) {
      if ((vb >> u) & 1u) {                              // (wavefront-uniform)
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)src, u);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(src >> 32), u);
        lds_load16(((uint64_t)hi << 32) | lo, tb + 2u * (uint32_t)trow(u));
      }
    }
  }
  if (sl < CC / 8) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      u32x2 x[4];
      int e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* row = rw + 4 * (4 * b + i) * kRawPitch;
        x[i] = *(const u32x2*)(row + 8 * sl);
        e[i] = (int)(int8_t)row[kD + kR + (sl >> 3)];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = ldexpf(1.0f, e[i]);
        u32x4 out;
        out[0] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16_scaled<false>(x[i][0], sc));
        out[1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16_scaled<true>(x[i][0], sc));
        out[2] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16_scaled<false>(x[i][1], sc));
        out[3] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16_scaled<true>(x[i][1], sc));
        if (!WIN || 4 * b + i < u_rec) *(u32x4*)(tw + trow(4 * b + i) + 8 * sl) = out;
      }
    }
  }
  {
    // lane l: rows u = l/8 and l/8 + 8, 16 B chunk l%8 of the 128 B rotary part
    const int c = sl & 7, u0 = sl >> 3;
    const u32x4 r0 = *(const u32x4*)(rw + 4 * u0 * kRawPitch + CC + 16 * c);
    const u32x4 r1 = *(const u32x4*)(rw + 4 * (u0 + 8) * kRawPitch + CC + 16 * c);
    if (!WIN || u0 < u_rec) *(u32x4*)(tw + trow(u0) + CC + 8 * c) = r0;
    if (!WIN || u0 + 8 < u_rec) *(u32x4*)(tw + trow(u0 + 8) + CC + 8 * c) = r1;
  }
  if (vb != 0xFFFFu) {                                   // rows without an item (uniform)
#pragma unroll
    for (int u = 0; u < kRows / 4; ++u)
      if (!((vb >> u) & 1u)) *(u32x4*)(tw + trow(u) + 8 * sl) = u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (WIN) __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the window rows have landed
}

// S^T (32 items x 32 heads) = K Q^T over the 512 channels: 32 MFMAs in one
// accumulation chain (TWO: two chains, even and odd channel steps, added at the end),
// K fragments (row l%32, 16 B at channel 16s + 8(l/32)) read kPf steps ahead;
// between(u) runs after every second MFMA (u = 0..15).  Two chains measure faster
// with fp8 entries and prepared queries (decode), slower with bf16 entries, and
// do not fit the registers of the fp8 raw-query variant.
constexpr int kPf = 4;
template <bool TWO, class F>
__device__ __forceinline__ void mx_scores(const __bf16* kt, const bf16x8* qf, f32x16& s_out, const F& between) {
  const int lane = threadIdx.x & 63;
  const __bf16* krow = kt + mx_row(lane & 31) * kPitch + 8 * (lane >> 5);
  f32x16 acc, acc1;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = acc1[v] = 0.0f;
  bf16x8 kf[kPf];
#pragma unroll
  for (int s = 0; s < kPf; ++s) kf[s] = *(const bf16x8*)(krow + 16 * s);
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    if (TWO && (s & 1)) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % kPf], qf[s], acc1, 0, 0, 0);
    else acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % kPf], qf[s], acc, 0, 0, 0);
    if (s + kPf < 32) kf[s % kPf] = *(const bf16x8*)(krow + 16 * (s + kPf));
    if (s & 1) between(s >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (TWO) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += acc1[v];
  }
  s_out = acc;
}

// O^T (256 channels in 8 blocks of 32 x 32 heads) += V^T P^T over the 64 items of a
// tile: for each 32-item half (pown: this wavefront's items, ppar: its partner's),
// two k-steps of 16 items x 8 channel blocks; V fragments (two transpose loads
// each) read kPf MFMAs ahead.
__device__ __forceinline__ void mx_pv(const __bf16* tile, int half, const bf16x8* pown, const bf16x8* ppar,
                                      f32x16* o) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int lane = threadIdx.x & 63, G = lane >> 4, i = lane & 15;
  const int col = 256 * half + 16 * (G & 1) + 4 * (i & 3);
  const __bf16* va0 = tile + mx_row(4 * (G >> 1) + (i >> 2)) * kPitch + col;      // items e, e + 8 of a
  const __bf16* vc0 = tile + mx_row(4 * (G >> 1) + (i >> 2) + 8) * kPitch + col;  // 16-item k-step
  // step n: item half ih = n >> 4 (0: own, 1: partner), k-step ks = (n >> 3) & 1, column block cb = n & 7
  auto rowbase = [&](int n) { return 32 * ((n >> 4) ? 1 - half : half) + 16 * ((n >> 3) & 1); };
  bf16x4 va[kPf], vc[kPf];
#pragma unroll
  for (int n = 0; n < kPf; ++n) {
    va[n] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + rowbase(n) * kPitch + 32 * (n & 7)));
    vc[n] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vc0 + rowbase(n) * kPitch + 32 * (n & 7)));
  }
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    bf16x8 vv;
    vv[0] = va[n % kPf][0]; vv[1] = va[n % kPf][1]; vv[2] = va[n % kPf][2]; vv[3] = va[n % kPf][3];
    vv[4] = vc[n % kPf][0]; vv[5] = vc[n % kPf][1]; vv[6] = vc[n % kPf][2]; vv[7] = vc[n % kPf][3];
    if (n + kPf < 32) {
      const int m = n + kPf;
      va[n % kPf] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + rowbase(m) * kPitch + 32 * (m & 7)));
      vc[n % kPf] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vc0 + rowbase(m) * kPitch + 32 * (m & 7)));
    }
    const bf16x8 pa = (n >> 4) ? ppar[(n >> 3) & 1] : pown[(n >> 3) & 1];
    o[n & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pa, o[n & 7], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O = 0, written by MFMAs (zero operands) so that the accumulators are only ever
// defined by MFMAs and stay in the accumulation registers across the tile loop.
__device__ __forceinline__ void mx_zero(f32x16* o) {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
  const f32x16 zc = {};
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, zc, 0, 0, 0);
}

// exp2 of the masked logits (times the head's factor qinv) against the reference, as
// bf16 P^T fragments; returns the fp32 sum.
__device__ __forceinline__ float mx_probs(const float* sv, float qinv, float m_run, bf16x8* pa) {
  float p[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[v], qinv, -m_run));
    pa[v >> 3][v & 7] = (__bf16)p[v];
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)                     // pairwise sum (short dependency chain)
#pragma unroll
    for (int v = 0; v < w; ++v) p[v] += p[v + w];
  return p[0];
}

// Queries of every (row, head) prepared once per row for rows whose items are
// split over several workgroups (qprep_head): one wavefront per (row, head).
__global__ void __launch_bounds__(256) attend_qprep_kernel(AttendArgs a) {
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= a.n_heads) return;
  qprep_head(a, blockIdx.x, h, threadIdx.x & 63);
}

// Units of an MFMA attention launch: n_rows x n_splits (split, row) pairs padded to a
// multiple of 8, times n_hg head groups (see attend_mx_kernel).
__host__ __device__ __forceinline__ int mx_unit_count(int n_rows, int n_hg, int n_splits) {
  return (n_rows * n_splits + 7) / 8 * 8 * n_hg;
}

// Dense numbering of the real (split, row) pairs of a decode launch of at most 64
// rows: pair q is split s of the k-th row, in row order, among the rows with more
// than s splits.  Like the padded numbering it is split-major, but it leaves no gaps,
// so the real units take the lowest workgroup ids and each XCD (block id mod 8) gets
// an even share of them whatever the rows' lengths.  Every wavefront finds the same
// answer on its own (lane = row; ballots, no LDS or barrier); *pos_r and *cnt_r
// receive the row's words as loaded.
__device__ __forceinline__ bool dense_pair(const AttendArgs& a, int q, int* split, int* r, int* pos_r,
                                           int* cnt_r) {
  const int lane = threadIdx.x & 63;
  int ns = 0, pw = 0, cw = 0;
  if (lane < a.n_rows) {
    pw = a.pos[lane];
    cw = a.mode == 0 ? a.cnt[lane] : 0;
    const int n = split_plan_count32(row_info_of(a, lane, pw, cw, false).total, a.split_min, a.split_div,
                                     a.split_cap);
    ns = n < a.max_splits ? n : a.max_splits;         // as n_splits_of: 1 .. max_splits
  }
  int rem = q;
  for (int s = 0; s < a.max_splits; ++s) {
    const uint64_t b = __ballot(ns > s);               // the rows of level s
    const int c = __popcll(b);
    if (rem < c) {
      // the rem-th set bit of b
      const bool hit = ((b >> lane) & 1ull) && __popcll(b & ((1ull << lane) - 1ull)) == rem;
      const int row = __ffsll((unsigned long long)__ballot(hit)) - 1;
      *split = s;
      *r = row;
      *pos_r = __builtin_amdgcn_readlane(pw, row);
      *cnt_r = __builtin_amdgcn_readlane(cw, row);
      return true;
    }
    rem -= c;
  }
  return false;                                        // past the last real pair
}

// MODE 0: CSA (the row's selected entries), 1: HCA (all of the row's entries);
// a compile-time copy of a.mode, so that the two attention kinds are distinct kernels.
// QP: the queries come prepared in a.q_prep, their RMSNorm factors in a.q_inv (no
// per-workgroup transform).
// DENSE (HCA decode launches only): the real units are numbered by dense_pair.
template <int KV_FMT, int MODE, bool QP, bool DENSE>
__global__ void __launch_bounds__(256) attend_mx_kernel(AttendArgs a) {
  a.mode = MODE;
  typedef MxCfg<KV_FMT> C;
  typedef MxShared<KV_FMT> Sh;
  __shared__ Sh sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = wave >> 1, half = wave & 1, partner = wave ^ 1;
  // Workgroups take units (split, row, head group of 64) with a static stride, so that
  // the work of a launch does not depend on scheduling.  The (split, row) pairs are
  // numbered split-major; unit u is head group (u % 8n_hg) / 8 of pair 8(u / 8n_hg) +
  // u % 8, so that the head groups of a pair, which read the same items, share u % 8:
  // the XCD of a workgroup (with a grid that is a multiple of 8).  The unit space is
  // padded to whole blocks of 8 pairs; padding units do nothing.
  // Decode launches of up to 64 rows whose padded unit space exceeds the CUs number the
  // pairs densely (dense_pair); the unit's row words then come from that search.
  const int n_hg = a.n_heads / 64, n_sp = a.split_min > 0 ? a.max_splits : 1;
  const int n_pairs = a.n_rows * n_sp;
  const int n_units = mx_unit_count(a.n_rows, n_hg, n_sp);
  constexpr bool dense = DENSE;
  int d_pos = 0, d_cnt = 0;
  auto unit_of = [&](int u, int* split, int* r, int* hg) {
    const int o = u % (8 * n_hg), p = u / (8 * n_hg) * 8 + (o & 7);
    *hg = o >> 3;
    if (dense) return dense_pair(a, p, split, r, &d_pos, &d_cnt);
    *split = p / a.n_rows;
    *r = p % a.n_rows;
    return p < n_pairs;
  };
  constexpr int CC = kD - kR;
  if constexpr (!QP)   // the query transform's factors (prepared queries have had them applied)
    for (int i = tid; i < kD; i += 256) sh.gain[i] = a.q_gain[i] * a.scale_log2;

  // Raw (or prepared) query rows (bf16 bits as B fragments: lane = head l%32, channels
  // 16s + 8(l/32) .. +7).  The next unit's rows are fetched early (after the last QK,
  // or after the tile loop), so their latency hides behind the unit's end.
  bf16x8 qf[32];
  float qf_inv = 1.0f;                                 // prepared rows: the row's RMSNorm factor
  int q_row = -1, q_hg = -1;                           // rows held in qf
  constexpr bool qp = QP;                              // queries come prepared (split rows)
  auto load_q = [&](int rr, int hh) {
    const int64_t qi = (int64_t)rr * a.n_heads + hh * 64 + 32 * pair + (lane & 31);
    const uint16_t* qrow = (qp ? a.q_prep : (const uint16_t*)a.q) + qi * kD + 8 * (lane >> 5);
    if constexpr (qp) qf_inv = a.q_inv[qi];
#pragma unroll
    for (int s = 0; s < 32; ++s) qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * s));
    q_row = rr;
    q_hg = hh;
  };
  // RMSNorm with gain, RoPE at t (table in sh.rope_cs), logit scale * log2(e), in place
  // and in one pass: the rows are stored without the norm's 1 / rms (x * gain * scale,
  // rotated), which is returned and applied to the head's logits instead (a per-head
  // factor commutes with the rotation and the dot products).
  auto transform_q = [&]() {
    float ss = 0.0f;
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int d0 = 16 * s + 8 * (lane >> 5);
      const f32x4 g0 = *(const f32x4*)(sh.gain + d0), g1 = *(const f32x4*)(sh.gain + d0 + 4);
      const u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(w[e] << 16);
        x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += x[e] * x[e];
        x[e] *= e < 4 ? g0[e] : g1[e - 4];
      }
      if (d0 >= CC) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int p = (d0 + e - CC) >> 1;
          const float c = sh.rope_cs[2 * p], sn = sh.rope_cs[2 * p + 1];
          const float x0 = x[e], x1 = x[e + 1];
          x[e] = x0 * c - x1 * sn;
          x[e + 1] = x0 * sn + x1 * c;
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[2 * e], (__bf16)x[2 * e + 1]});
      qf[s] = __builtin_bit_cast(bf16x8, o);
    }
    ss += __shfl_xor(ss, 32, 64);
    return 1.0f / sqrtf(ss / (float)kD + a.eps);
  };

  constexpr int kPrologueTiles = C::kFp8 ? 2 : 1;
  // bf16 prefill: the sequence's page-table row in LDS (see kLdsPages)
  const int32_t* pt_l = nullptr;
  if (!C::kFp8 && a.seq_fixed >= 0 && a.kv.max_pages > 0 && a.kv.max_pages <= kLdsPages) {   // (uniform)
    for (int i = tid; i < a.kv.max_pages; i += 256) sh.pt[i] = a.kv.page_table[(int64_t)a.seq_fixed * a.kv.max_pages + i];
    __syncthreads();
    pt_l = sh.pt;
  }
  float m_force = kNoMax;                              // != kNoMax: recompute the unit with this reference
  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
  int split, r, hg;
  if (!unit_of(unit, &split, &r, &hg)) continue;       // padding (workgroup-uniform)
  const RowInfo ri = dense ? row_info_of(a, r, d_pos, d_cnt) : row_info(a, r);
  const int ns = n_splits_of(a, ri.total);
  if (split >= ns) continue;
  int j0, j1;
  split_range(a, ri.total, split, &j0, &j1);
  j1 = j1 - j0 > kMaxItems ? j0 + kMaxItems : j1;      // (the plan never exceeds the item table)
  const int ntiles = (j1 - j0 + kRows - 1) / kRows;
  const int head0 = hg * 64 + 32 * pair;               // first head of this pair
  const int hl = lane & 31;                            // head (within the block) of this lane's S^T column

  // ---- prologue.  Query loads (unless prefetched) go out right behind the item
  // table's last dependent loads (ahead of them they would delay that round trip):
  // their transfer overlaps it, and being older than the tile loads, waiting for them
  // never waits for a tile.
  if (!qp && tid < kR / 2) {                           // (the table serves the transform and de-rotation)
    // angle t * theta_p with theta_p = rope_step^p (binary powering in fp64), taken in
    // revolutions and reduced exactly in fp64; the hardware sin / cos take revolutions
    double th = 1.0, bp = a.rope_step;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      th = ((tid >> k) & 1) ? th * bp : th;
      bp *= bp;
    }
    const double rev = (double)ri.t * th * 0.15915494309189535;   // 1 / (2 pi)
    const float fr = (float)(rev - floor(rev));
    sh.rope_cs[2 * tid] = __builtin_amdgcn_cosf(fr);
    sh.rope_cs[2 * tid + 1] = __builtin_amdgcn_sinf(fr);
  }
  const int n_tab = (j1 - j0) < kMaxItems ? (j1 - j0) : kMaxItems;
  if (q_row != r || q_hg != hg)   // (workgroup-uniform; two straight-line copies, so that
                                  // the wait for the table's loads does not wait for the queries)
    mx_item_table<MODE>(a, ri, r, j0, n_tab, sh.items, pt_l, [&]() { load_q(r, hg); });
  else
    mx_item_table<MODE>(a, ri, r, j0, n_tab, sh.items, pt_l, []() {});
  // a valid, finite row used as the source of loads for rows without an item: the window token at t
  const uint8_t* dummy = (const uint8_t*)a.win + ((int64_t)ri.win_seq * a.W + ri.t % a.W) * kD * 2;
  __syncthreads();
  // vmcnt(0), as a builtin the compiler understands: the query loads (older than the
  // item-table loads just awaited) are complete, so no wait for them is placed inside
  // the MFMA loops, where the tile loads in flight would make it a real stall
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  for (int t = 0; t < kPrologueTiles; ++t) {
    MxIssue<KV_FMT> is;
    is.prepare(a, j0, j1, t, t, sh, dummy, t < ntiles);
    is.all();
  }

  float qinv = qf_inv;                                 // logit factor of the lane's head (1 / rms)
  if constexpr (!qp) qinv = transform_q();
  q_row = -1;                                          // qf now holds transformed queries

  // Softmax reference: m_run is set by the first tile with a valid item (O is still
  // zero then) and never moves afterwards; probabilities relative to it stay below
  // 2^kBump, far inside fp32/bf16 range, unless a later logit exceeds it by more
  // than kBump.  That (practically unreachable) case sets `redo` and the unit is
  // recomputed with the exact maximum m_true seen on the first pass, so the loop
  // never rescales O and the accumulators never leave their registers.
  constexpr float kBump = 60.0f;
  f32x16 oacc[8];
  mx_zero(oacc);
  float m_run = m_force, l_part = 0.0f, m_loc = kNoMax;   // m_loc: max logit of this lane's items
  bool redo = false;
  for (int tile = 0; tile < ntiles; ++tile) {
    const int st = tile & 1;
    if constexpr (C::kFp8) {
      if (tile + 1 < ntiles) __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    __syncthreads();                                   // tile landed for every wavefront
    const u32x4 vw = *(const u32x4*)sh.valid[st];      // (fp8: read before the stage is refilled)
    const __bf16* tl;
    MxIssue<KV_FMT> is;
    if constexpr (C::kFp8) {
      const int jt = j0 + tile * kRows;
      if (jt + kRows > ri.n_c)                         // (workgroup-uniform) the tile reaches the window
        mx_convert<true>(a, sh.ring[st], sh.valid[st], sh.items, jt, j0, ri.n_c, sh.tile);
      else
        mx_convert<false>(a, sh.ring[st], sh.valid[st], sh.items, jt, j0, ri.n_c, sh.tile);
      __syncthreads();
      is.prepare(a, j0, j1, tile + 2, st, sh, dummy, tile + 2 < ntiles);
      tl = sh.tile;
    } else {
      is.prepare(a, j0, j1, tile + 1, st ^ 1, sh, dummy, tile + 1 < ntiles);
      tl = (const __bf16*)sh.ring[st];
    }
    // the next tile's row loads go out between the QK MFMAs (one row after every
    // second MFMA), so that their issue overlaps the matrix work
    f32x16 s;
    constexpr bool kTwoChains = C::kFp8 && qp;
    if (is.on)
      mx_scores<kTwoChains>(tl + 32 * half * kPitch, qf, s, [&](int u) { is.row(u); });
    else
      mx_scores<kTwoChains>(tl + 32 * half * kPitch, qf, s, [](int) {});
    if (!C::kFp8 && !dense && tile == ntiles - 1 && unit + (int)gridDim.x < n_units) {
      int s2, r2, h2;                                  // prefetch the next unit's queries (bf16:
      if (unit_of(unit + gridDim.x, &s2, &r2, &h2)) load_q(r2, h2);   // right after the last QK)
    }
    float sv[16];
    float mx = -INFINITY;
    if ((vw[0] & vw[1] & vw[2] & vw[3] & 0xFFFFu) == 0xFFFFu) {      // every row holds an item
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = s[v];
        mx = fmaxf(mx, sv[v]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = (vw[v & 3] >> (8 * half + 2 * (v >> 2) + (lane >> 5))) & 1u;
        sv[v] = ok ? s[v] : -INFINITY;
        mx = fmaxf(mx, sv[v]);
      }
    }
    mx *= qinv;                                        // (sv: logits before the head's factor)
    // a logit above the reference by more than kBump anywhere in the workgroup?  (Any
    // lane's own maximum will do: no per-head maximum is formed on the common path.)
    const bool bump = __any(mx > m_run + kBump);
    m_loc = fmaxf(m_loc, mx);
    bf16x8 pown[2];
    float psum = mx_probs(sv, qinv, m_run, pown);
    *(bf16x8*)&sh.pex[wave][lane][0] = pown[0];
    *(bf16x8*)&sh.pex[wave][lane][1] = pown[1];
    if (lane == 0) sh.bump[wave] = bump;
    __syncthreads();
    // everything the exchange delivers, read at once
    const i32x4 bumps = *(const i32x4*)sh.bump;
    bf16x8 ppar[2];
    ppar[0] = *(const bf16x8*)&sh.pex[partner][lane][0];
    ppar[1] = *(const bf16x8*)&sh.pex[partner][lane][1];
    if (__builtin_expect(bumps[0] | bumps[1] | bumps[2] | bumps[3], 0)) {   // workgroup-uniform
      if (m_run == kNoMax) {
        // first tile with valid items (the same tile for every head): the reference is the
        // pair's maximum logit of each head over this tile
        const float tmax = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (lane < 32) sh.tmx[wave][lane] = tmax;
        __syncthreads();                               // every wavefront has read the exchange
        m_run = fmaxf(tmax, sh.tmx[partner][hl]);
        psum = mx_probs(sv, qinv, m_run, pown);
        *(bf16x8*)&sh.pex[wave][lane][0] = pown[0];
        *(bf16x8*)&sh.pex[wave][lane][1] = pown[1];
        __syncthreads();
        ppar[0] = *(const bf16x8*)&sh.pex[partner][lane][0];
        ppar[1] = *(const bf16x8*)&sh.pex[partner][lane][1];
      } else {
        redo = true;
      }
    }
    l_part += psum;
    mx_pv(tl, half, pown, ppar, oacc);
  }

  if (C::kFp8 && !dense && unit + (int)gridDim.x < n_units) {   // prefetch the next unit's queries (fp8:
    int s2, r2, h2;                                    // after the loop, whose top wait the
    if (unit_of(unit + gridDim.x, &s2, &r2, &h2)) load_q(r2, h2);   // compiler cannot see)
  }
  if (__builtin_expect(redo && m_force == kNoMax, 0)) {  // workgroup-uniform
    // a logit overflowed the reference: recompute the unit against the exact maximum
    // of each head over the pair's items
    const float mt = fmaxf(m_loc, __shfl_xor(m_loc, 32, 64));
    if (lane < 32) sh.tmx[wave][lane] = mt;
    __syncthreads();
    m_force = fmaxf(mt, sh.tmx[partner][hl]);
    unit -= gridDim.x;
    __syncthreads();                                   // every wavefront is done with the ring
    continue;
  }
  m_force = kNoMax;

  // ---- epilogue: per-head sum over the pair's items
  const float l_own = l_part + __shfl_xor(l_part, 32, 64);
  if (lane < 32) sh.lsum[wave][lane] = l_own;
  __syncthreads();                                     // also: every wavefront is done with the tiles
  const float l_tot = l_own + sh.lsum[partner][hl];
  const int c0 = 256 * half;                           // first channel of this wavefront's O
  const bool split_out = a.split_min > 0;
  if (split_out) {
    // split partials go out in the accumulator layout (the combine kernel reads it):
    // per (row, split, head group) a block [pair][half][cb][v/4][lane][v%4] of fp32
    // (or bf16), so that each store instruction writes 1 KB (512 B) contiguous
    const int64_t pbase = ((int64_t)r * a.max_splits + split) * a.n_heads + head0;
    if (half == 0 && lane < 32) {
      a.part_ml[2 * (pbase + hl)] = m_run;
      a.part_ml[2 * (pbase + hl) + 1] = l_tot;
    }
    const int64_t blk = (((int64_t)r * a.max_splits + split) * n_hg + hg) * (64 * kD) +
                        (pair * 2 + half) * (8 * 4 * 64 * 4) + 4 * lane;   // element offset
    if (a.part_bf16) {   // (uniform) 8 B per lane: each store instruction writes 512 B contiguous
      uint16_t* pb = (uint16_t*)a.part_o + blk;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          u32x2 w;
          w[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)oacc[cb][4 * vq], (__bf16)oacc[cb][4 * vq + 1]});
          w[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)oacc[cb][4 * vq + 2], (__bf16)oacc[cb][4 * vq + 3]});
          *(u32x2*)(pb + (cb * 4 + vq) * 256) = w;
        }
    } else {
      float* pf = a.part_o + blk;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          *(f32x4*)(pf + (cb * 4 + vq) * 256) =
              f32x4{oacc[cb][4 * vq], oacc[cb][4 * vq + 1], oacc[cb][4 * vq + 2], oacc[cb][4 * vq + 3]};
    }
    __syncthreads();                                   // the next unit reuses the LDS
    continue;
  }
  // The lane's O^T elements are its own head's: scaled by the head's factor, the
  // rotary channels 448..511 rotated by R_{-t} within the lane (pairs (2p, 2p + 1)
  // are elements v, v + 1 with v even), and stored as runs of 4 channels (8 B bf16 or
  // 16 B fp32; lanes l and l + 32 write adjacent runs).
  const float sk_own = a.sink[head0 + hl] * kLog2e;
  const float M_own = fmaxf(m_run, sk_own);
  const float den_own = l_tot * __builtin_amdgcn_exp2f(m_run - M_own) + __builtin_amdgcn_exp2f(sk_own - M_own);
  const float f_own = __builtin_amdgcn_exp2f(m_run - M_own) / den_own;
  if (a.lse && half == 0 && lane < 32) a.lse[(int64_t)r * a.n_heads + head0 + hl] = (M_own + log2f(den_own)) / kLog2e;
  const int64_t ob = ((int64_t)r * a.n_heads + head0 + hl) * kD + c0 + 4 * (lane >> 5);
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = oacc[cb][4 * vq + e] * f_own;
      if (c0 + 32 * cb >= CC) {                        // (wavefront-uniform)
        const int p0 = (c0 + 32 * cb + 8 * vq + 4 * (lane >> 5) - CC) >> 1;
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const float c = sh.rope_cs[2 * (p0 + e / 2)], sn = sh.rope_cs[2 * (p0 + e / 2) + 1];
          const float x0 = x[e], x1 = x[e + 1];
          x[e] = x0 * c + x1 * sn;
          x[e + 1] = x1 * c - x0 * sn;
        }
      }
      const int64_t o = ob + 32 * cb + 8 * vq;
      if (a.out_fmt == CA_F32) {
        *(f32x4*)((float*)a.out + o) = x;
      } else {
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[0], (__bf16)x[1]});
        w[1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[2], (__bf16)x[3]});
        *(u32x2*)((uint16_t*)a.out + o) = w;
      }
    }
  }
  __syncthreads();                                     // the next unit reuses the LDS
  }
}

// ======================================================================== dispatch
int attend_mfma_max_items() { return kMaxItems; }

// Compute units of the current device (one persistent attention workgroup each).
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool attend_mfma_supported(const AttendArgs& a) {
  // items are addressed by 31-bit pool record index or window row (the host keeps both below
  // 2^31 - 1; checked again here)
  const bool fits = ((int64_t)a.kv.n_pages << a.kv.page_shift) < 0x7FFFFFFF &&
                    (int64_t)a.W * (a.seq_fixed >= 0 ? 1 : a.n_rows) < 0x7FFFFFFF;
  return a.D == kD && a.R == kR && a.n_heads % 64 == 0 && a.q_fmt == CA_BF16 && a.win_fmt == CA_BF16 &&
         (a.kv.fmt == CA_BF16 || a.kv.fmt == CA_FP8MIX) && fits;
}

hipError_t launch_attend(const AttendArgs& args, hipStream_t st, bool q_prepared) {
  if (args.n_rows == 0) return hipSuccess;
  AttendArgs a = args;
  a.part_acc = attend_mfma_supported(a) ? 1 : 0;
  a.part_bf16 = a.out_fmt == CA_BF16 ? 1 : 0;   // partials no finer than the output
  const int splits = a.split_min > 0 ? a.max_splits : 1;
  hipEvent_t ev0, ev1;
  timer_events(a.mode == 0 ? CA_TIMED_CSA_ATTEND : CA_TIMED_HCA_ATTEND, st, &ev0, &ev1);
  if (attend_mfma_supported(a)) {
    if (a.q_prep != nullptr && !q_prepared)
      hipLaunchKernelGGL(attend_qprep_kernel, dim3(a.n_rows, a.n_heads / 4), dim3(256), 0, st, a);
    // Persistent workgroups (one per CU) for prefill.  Split (decode) launches take one
    // workgroup per unit up to 4 per CU: the unit space is every row's largest split count,
    // numbered split-major (split 0 of every row and head group first), so the real units
    // of a batch with short rows take the low workgroup ids that are dispatched first, and
    // units a row does not have exit at once (a static stride would stack two real units
    // on some workgroups).
    const long units = mx_unit_count(a.n_rows, a.n_heads / 64, splits);
    const long cap = splits > 1 && units <= 4L * cu_count() ? units : cu_count();
    // Workgroups past the first one per CU start only as earlier ones finish, so when the
    // padded unit space of a decode launch exceeds the CUs, rows with fewer splits than
    // the most would leave gaps below that line and push real units above it: number the
    // real units densely instead (dense_pair; up to 64 rows, one per lane).  HCA only:
    // its rows' lengths follow their positions, while CSA rows from m * k tokens on all
    // hold k + n_win items, so their padded numbering has no gaps (and the search would
    // only add its cost).
    a.dense_units = a.mode == 1 && a.pos != nullptr && splits > 1 && a.n_rows <= 64 && units > cu_count() ? 1 : 0;
    dim3 grid((unsigned)(units < cap ? units : cap));
    const bool qp = a.q_prep != nullptr;
#define CA_MX(F, M, Q, DN) CA_LAUNCH((attend_mx_kernel<F, M, Q, DN>), grid, dim3(256), 0, st, ev0, ev1, a)
    if (a.kv.fmt == CA_FP8MIX) {
      if (a.mode == 0) {
        if (qp) CA_MX(CA_FP8MIX, 0, true, false);
        else CA_MX(CA_FP8MIX, 0, false, false);
      } else if (a.dense_units) {
        if (qp) CA_MX(CA_FP8MIX, 1, true, true);
        else CA_MX(CA_FP8MIX, 1, false, true);
      } else {
        if (qp) CA_MX(CA_FP8MIX, 1, true, false);
        else CA_MX(CA_FP8MIX, 1, false, false);
      }
    } else {
      if (a.mode == 0) {
        if (qp) CA_MX(CA_BF16, 0, true, false);
        else CA_MX(CA_BF16, 0, false, false);
      } else if (a.dense_units) {
        if (qp) CA_MX(CA_BF16, 1, true, true);
        else CA_MX(CA_BF16, 1, false, true);
      } else {
        if (qp) CA_MX(CA_BF16, 1, true, false);
        else CA_MX(CA_BF16, 1, false, false);
      }
    }
#undef CA_MX
  } else {
    dim3 grid(a.n_rows, a.n_heads, splits);
    switch (a.D / 64) {
      case 1: CA_LAUNCH(attend_generic_kernel<1>, grid, dim3(64), 0, st, ev0, ev1, a); break;
      case 2: CA_LAUNCH(attend_generic_kernel<2>, grid, dim3(64), 0, st, ev0, ev1, a); break;
      case 4: CA_LAUNCH(attend_generic_kernel<4>, grid, dim3(64), 0, st, ev0, ev1, a); break;
      case 8: CA_LAUNCH(attend_generic_kernel<8>, grid, dim3(64), 0, st, ev0, ev1, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.split_min <= 0) return e;
  if (a.part_acc) {
    const dim3 grid(a.n_rows, (a.n_heads / 64) * 16);
    if (a.part_bf16) hipLaunchKernelGGL(attend_combine_acc_kernel<true>, grid, dim3(512), 0, st, a);
    else hipLaunchKernelGGL(attend_combine_acc_kernel<false>, grid, dim3(512), 0, st, a);
  } else {
    const int hpb = 512 / (a.D / 4);                   // heads per combine workgroup
    const dim3 grid(a.n_rows, (a.n_heads + hpb - 1) / hpb);
    if (a.part_bf16) hipLaunchKernelGGL(attend_combine_kernel<true>, grid, dim3(512), 0, st, a);
    else hipLaunchKernelGGL(attend_combine_kernel<false>, grid, dim3(512), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ca
