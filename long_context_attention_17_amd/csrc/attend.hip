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
constexpr int kTile = 32;          // items per tile
constexpr int kPitch = kD + 8;     // bf16 elements per LDS row (16 B pad against bank conflicts)

struct TileRegs {
  u32x4 raw[8];
  int kind[8];   // 0: skipped item (zeros), 1: bf16 row (entry or window), 2: fp8-mixed entry
  float scale[8];
};

// Issue the global loads of tile `j_begin .. j_begin+31` of this row.
// Wave w handles items w, w+4, ..., lane q its 16-byte chunk q of the item.
template <int KV_FMT>
__device__ __forceinline__ void tile_load(const AttendArgs& a, const RowInfo& ri, int r, int j_begin, int j_end,
                                          TileRegs& tr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int j = j_begin + wave + 4 * u;
    bool is_win = false;
    const uint8_t* p = j < j_end ? item_ptr(a, ri, r, j, &is_win) : nullptr;
    tr.kind[u] = p == nullptr ? 0 : ((KV_FMT == CA_FP8MIX && !is_win) ? 2 : 1);
    tr.raw[u] = u32x4{0, 0, 0, 0};
    tr.scale[u] = 1.0f;
    if (tr.kind[u] == 1) {
      tr.raw[u] = ((const u32x4*)p)[lane];
    } else if (tr.kind[u] == 2) {
      if (lane < 28) {
        tr.raw[u] = ((const u32x4*)p)[lane];                         // 16 content codes
        tr.scale[u] = ldexpf(1.0f, (int)(int8_t)p[kD + 64 + (lane >> 2)]);   // exponents after codes + rope
      } else if (lane < 36) {
        tr.raw[u] = ((const u32x4*)(p + 448))[lane - 28];            // 8 rotary bf16
      }
    }
  }
}

// Dequantize / copy the loaded tile into LDS buffer `kt`, and its item mask.
__device__ __forceinline__ void tile_store(__bf16* kt, int* valid, const TileRegs& tr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int it = wave + 4 * u;
    __bf16* row = kt + it * kPitch;
    if (tr.kind[u] == 2) {
      if (lane < 28) {
        bf16x8 lo, hi;
        const u32x4 w = tr.raw[u];
        const float sc = tr.scale[u];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          bf16x2 a0 = e4m3x2_to_bf16_scaled<false>(w[2 * k], sc), a1 = e4m3x2_to_bf16_scaled<true>(w[2 * k], sc);
          bf16x2 b0 = e4m3x2_to_bf16_scaled<false>(w[2 * k + 1], sc), b1 = e4m3x2_to_bf16_scaled<true>(w[2 * k + 1], sc);
          bf16x8& dst = k == 0 ? lo : hi;
          dst[0] = a0[0]; dst[1] = a0[1]; dst[2] = a1[0]; dst[3] = a1[1];
          dst[4] = b0[0]; dst[5] = b0[1]; dst[6] = b1[0]; dst[7] = b1[1];
        }
        *(bf16x8*)(row + 16 * lane) = lo;
        *(bf16x8*)(row + 16 * lane + 8) = hi;
      } else if (lane < 36) {
        *(u32x4*)(row + 448 + 8 * (lane - 28)) = tr.raw[u];
      }
    } else {
      *(u32x4*)(row + 8 * lane) = tr.raw[u];   // bf16 row, or zeros for a skipped item
    }
    if (lane == 0) valid[it] = tr.kind[u] != 0;
  }
}

template <int KV_FMT>
__global__ void __launch_bounds__(256) attend_mfma_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 ktile[2][kTile * kPitch];
  __shared__ int valid[2][kTile];

  const int r = blockIdx.x, hg = blockIdx.y, split = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

  TileRegs tr;
  if (ntiles > 0) tile_load<KV_FMT>(a, ri, r, j0, j1, tr);

  // ---- query prologue: RMSNorm, gain, RoPE at t, to bf16 B-operand fragments
  bf16x8 qreg[16];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)r * a.n_heads + head_s) * kD;
    float qf[16][8];
    float ss = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      u32x4 w = *(const u32x4*)(qrow + 32 * kb + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[kb][2 * e] = __uint_as_float(w[e] << 16);
        qf[kb][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += qf[kb][e] * qf[kb][e];
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float inv = 1.0f / sqrtf(ss / (float)kD + a.eps);
    const int C = kD - a.R;
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int d = 32 * kb + 8 * g + e;
        qf[kb][e] *= inv * a.q_gain[d];
      }
      if (32 * kb + 8 * g + 8 > C) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          int d = 32 * kb + 8 * g + e;
          if (d >= C) {
            float s, c;
            rope_sincos((double)ri.t, (d - C) >> 1, a.R, a.base, &s, &c);
            float x0 = qf[kb][e], x1 = qf[kb][e + 1];
            qf[kb][e] = x0 * c - x1 * s;
            qf[kb][e + 1] = x0 * s + x1 * c;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[kb][e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(qf[kb][e]));
    }
  }

  f32x4 oacc[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) oacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_part = 0.0f;

  if (ntiles > 0) tile_store(ktile[0], valid[0], tr);
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int jb = j0 + tile * kTile;
    if (tile + 1 < ntiles) tile_load<KV_FMT>(a, ri, r, jb + kTile, j1, tr);
    const __bf16* kt = ktile[buf];

    // S^T = K Q^T : two 16-item blocks, contraction over 512 dims
    f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 16; ++kb) {
      bf16x8 k0 = *(const bf16x8*)(kt + li * kPitch + 32 * kb + 8 * g);
      bf16x8 k1 = *(const bf16x8*)(kt + (16 + li) * kPitch + 32 * kb + 8 * g);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[kb], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[kb], s1, 0, 0, 0);
    }
    // lane: head li, items 4g+v (block 0) and 16+4g+v (block 1)
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sv[v] = valid[buf][4 * g + v] ? s0[v] * a.scale_log2 : -INFINITY;
      sv[4 + v] = valid[buf][16 + 4 * g + v] ? s1[v] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, fmaxf(sv[v], sv[4 + v]));
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.0f;
    bf16x8 pa;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = __builtin_bit_cast(__bf16, (uint16_t)0);
    } else {
      alpha = exp2f(m_run - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float p = exp2f(sv[e] - m_new);
        psum += p;
        pa[e] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(p));
      }
      l_part = l_part * alpha + psum;
      m_run = m_new;
    }
    // O rows held by this lane are heads 4g+v: fetch their rescale factors
    float al[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) al[v] = __shfl(alpha, 4 * g + v, 64);

    // O += P V ; V^T fragments via LDS transpose loads in the same item order
    const int vrow = 4 * g + (li >> 2), vcol = 4 * (li & 3);
    const __bf16* vbase = kt + vrow * kPitch + vcol;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
      bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase + 16 * cb));
      bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase + 16 * kPitch + 16 * cb));
      bf16x8 vv;
      vv[0] = va[0]; vv[1] = va[1]; vv[2] = va[2]; vv[3] = va[3];
      vv[4] = vb[0]; vv[5] = vb[1]; vv[6] = vb[2]; vv[7] = vb[3];
#pragma unroll
      for (int v = 0; v < 4; ++v) oacc[cb][v] *= al[v];
      oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vv, oacc[cb], 0, 0, 0);
    }
    if (tile + 1 < ntiles) tile_store(ktile[buf ^ 1], valid[buf ^ 1], tr);
    __syncthreads();
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
  const int C = kD - a.R;
  float rs[4], rc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {   // the 4 rotary column blocks 28..31 (dims 448..511 when R = 64)
    int d = 16 * (28 + q) + li;
    rs[q] = 0.0f;
    rc[q] = 1.0f;
    if (d >= C) rope_sincos((double)ri.t, (d - C) >> 1, a.R, a.base, &rs[q], &rc[q]);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t obase = ((int64_t)r * a.n_heads + head_base + 4 * g + v) * kD;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float x = oacc[cb][v] * fv[v];
      if (cb >= 28) {
        float other = __shfl_xor(x, 1, 64);
        int d = 16 * cb + li;
        if (d >= C) {
          float s = rs[cb - 28], c = rc[cb - 28];
          x = (li & 1) ? x * c - other * s : x * c + other * s;
        }
      }
      if (a.out_fmt == CA_F32) ((float*)a.out)[obase + 16 * cb + li] = x;
      else ((uint16_t*)a.out)[obase + 16 * cb + li] = f32_to_bf16_bits(x);
    }
  }
}

// ======================================================================== dispatch
bool attend_mfma_supported(const AttendArgs& a) {
  return a.D == kD && a.R == 64 && a.n_heads % 64 == 0 && a.q_fmt == CA_BF16 &&
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
