// Sequence compressors (CSA overlapping 2m softmax pooling, HCA disjoint
// pooling), the entry epilogue (RMSNorm -> partial RoPE -> record encode), the
// decode-time tail ring, and the sliding-window append.
//
// dsv4 book Ch.5 "The four compression projections", "Coordinate-wise softmax
// pooling", "Receptive field versus compression stride", "Decode-time cache
// state"; Ch.7 "HCA's 128:1 non-overlapping compressor", "The 128-token
// uncompressed sliding window", "Query and KV RMSNorm", "Partial RoPE and
// output de-rotation"; Ch.8 "V4 compressed-entry payload".
//
// Work layout: one workgroup per entry (or window token), one thread per
// channel; blockDim = dim rounded up to a multiple of 64, so every 64-channel
// content tile of a mixed record is exactly one wavefront and its amax is a
// wavefront reduction.  These kernels read each projection row once and are
// bound by HBM reads of the rows; they are a small share of any step.
#include "common.h"
#include "kernels.h"
#include "qprep.h"

namespace ca {

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
  for (int i = 1; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// RMSNorm (when gain != nullptr) then rotation of the last R channels at
// position `pos`.  Thread j holds channel j (x is ignored for j >= D).
__device__ float norm_rope(float x, int j, int D, int R, const float* gain, float eps, bool rope, double pos,
                           double base, float* red) {
  bool act = j < D;
  if (gain != nullptr) {
    float ss = block_sum(act ? x * x : 0.0f, red);
    float inv = 1.0f / sqrtf(ss / (float)D + eps);
    x = act ? x * inv * gain[j] : 0.0f;
  }
  if (rope && R > 0) {
    float other = __shfl_xor(x, 1, 64);  // pair partner (pairs start at even channels)
    if (act && j >= D - R) {
      int p = (j - (D - R)) >> 1;
      float s, c;
      rope_sincos(pos, p, R, base, &s, &c);
      x = (j & 1) ? other * s + x * c : x * c - other * s;
    }
  }
  return x;
}

// Encode channel j of entry i of sequence `seq` into the pool.
__device__ void store_record(const CacheView& cv, int seq, int64_t i, float x, int j, float* red) {
  const int D = cv.dim, R = cv.rope;
  bool act = j < D;
  uint8_t* page = cv.page_of(seq, i);
  int slot = cv.slot_of(i);
  if (cv.fmt == CA_FP8MIX) {
    const int C = D - R;
    // one wavefront == one 64-channel content tile
    float amax = wave_max((act && j < C) ? fabsf(x) : 0.0f);
    if (page == nullptr || !act) return;
    uint8_t* rec = page + slot * cv.stride;
    if (j < C) {
      int e = pow2_exponent(amax);
      rec[j] = (uint8_t)e4m3_encode(ldexpf(x, -e));
      if ((j & 63) == 0) rec[C + 2 * R + (j >> 6)] = (uint8_t)(int8_t)e;
    } else {
      ((uint16_t*)(rec + C))[j - C] = f32_to_bf16_bits(x);
    }
  } else if (cv.fmt == CA_E4M3) {
    float amax = block_max(act ? fabsf(x) : 0.0f, red);
    if (page == nullptr || !act) return;
    int e = pow2_exponent(amax);
    page[(int64_t)slot * D + j] = (uint8_t)e4m3_encode(ldexpf(x, -e));
    if (j == 0) ((float*)(page + ((int64_t)D << cv.page_shift)))[slot] = ldexpf(1.0f, e);
  } else if (cv.fmt == CA_FP4) {
    // a 32-channel block is half a wavefront (D % 32 == 0): its maximum, the
    // block exponent, then channel pairs (2c, 2c+1) packed into byte c
    float amax = act ? fabsf(x) : 0.0f;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const int e = fp4_block_exponent(amax);
    const uint32_t code = e2m1_encode(ldexpf(x, -e));
    const uint32_t odd = __shfl_xor(code, 1, 64);
    if (page == nullptr || !act) return;
    if ((j & 1) == 0) page[(int64_t)slot * (D / 2) + (j >> 1)] = (uint8_t)(code | (odd << 4));
    if ((j & 31) == 0) page[((int64_t)(D / 2) << cv.page_shift) + (int64_t)slot * (D / 32) + (j >> 5)] = (uint8_t)(e + 127);
  } else if (cv.fmt == CA_BF16) {
    if (page && act) ((uint16_t*)(page + slot * cv.stride))[j] = f32_to_bf16_bits(x);
  } else {
    if (page && act) ((float*)(page + slot * cv.stride))[j] = x;
  }
}

// Online softmax-weighted sum over pooled source positions (one channel).
struct Pool1 {
  float mx = -INFINITY, den = 0.0f, num = 0.0f;
  __device__ __forceinline__ void add(float z, float c) {
    if (z > mx) {
      float s = __expf(mx - z);
      den *= s;
      num *= s;
      mx = z;
    }
    float w = __expf(z - mx);
    den += w;
    num += w * c;
  }
  __device__ __forceinline__ float value() const { return num / den; }
};

__global__ void compress_prefill_kernel(CacheView cv, int seq, int m, int overlap, int in_fmt, const void* Ca,
                                        const void* Za, const void* Cb, const void* Zb, const float* Ba,
                                        const float* Bb, const float* gain, float eps, int apply_rope,
                                        double base, int64_t i0, int64_t t0) {
  __shared__ float red[16];
  const int D = cv.dim, j = threadIdx.x;
  const int64_t i = i0 + blockIdx.x;                   // entry; row index = position - t0
  float x = 0.0f;
  if (j < D) {
    Pool1 acc;
    for (int t = 0; t < m; ++t) {
      int64_t row = (int64_t)m * i + t - t0;
      acc.add(load_act(Za, in_fmt, row * D + j) + Ba[t * D + j], load_act(Ca, in_fmt, row * D + j));
    }
    if (overlap && i > 0) {
      for (int t = 0; t < m; ++t) {
        int64_t row = (int64_t)m * (i - 1) + t - t0;
        acc.add(load_act(Zb, in_fmt, row * D + j) + Bb[t * D + j], load_act(Cb, in_fmt, row * D + j));
      }
    }
    x = acc.value();
  }
  x = norm_rope(x, j, D, cv.rope, gain, eps, apply_rope != 0, (double)m * (double)i, base, red);
  store_record(cv, seq, i, x, j, red);
}

// Adds positions u = 0 .. m-1 of entry e to acc, in order, for channel j: logit
// z_arr[u] + B[u], value c_arr[u] from the tail ring (position p of the sequence in
// slot p % span, narr arrays of D floats per slot; span is m or 2m, so the m positions
// of an entry sit in the consecutive slots from (m e) % span).  BATCH positions at a
// time, every load of a batch issued before the first is used (positions past m
// re-read u = m - 1 and are not added).
template <int BATCH>
__device__ __forceinline__ void pool_positions(Pool1& acc, const float* ring, int m, int span, int narr, int D, int j,
                                               int64_t e, int c_arr, int z_arr, const float* B) {
  const float* first = ring + (int64_t)(((int64_t)m * e) % span) * narr * D;
  for (int u0 = 0; u0 < m; u0 += BATCH) {
    float z[BATCH], c[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      const int u = u0 + q < m ? u0 + q : m - 1;
      const float* slot = first + (int64_t)u * narr * D;
      z[q] = slot[z_arr * D + j] + B[u * D + j];
      c[q] = slot[c_arr * D + j];
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q)
      if (u0 + q < m) acc.add(z[q], c[q]);
  }
}

// Tail ring: tail[b, slot, a, ch] (float32), narr arrays per slot.
// Decode-time compressor step of sequence b (thread j = channel j; every thread of
// the block takes part, channels j >= D hold nothing).
__device__ __forceinline__ void compress_decode_row(const CacheView& cv, int m, int overlap, int in_fmt,
                                                    const void* new_rows, const int32_t* pos, float* tail,
                                                    const float* Ba, const float* Bb, const float* gain, float eps,
                                                    int apply_rope, double base, int b, int j, float* red) {
  const int D = cv.dim;
  const int narr = overlap ? 4 : 2;
  const int span = overlap ? 2 * m : m;
  const int t = pos[b];
  float* ring = tail + (int64_t)b * span * narr * D;
  if (j < D && t >= 0) {
    for (int a = 0; a < narr; ++a)
      ring[((int64_t)(t % span) * narr + a) * D + j] = load_act(new_rows, in_fmt, ((int64_t)b * narr + a) * D + j);
  }
  if (t < 0 || (t + 1) % m != 0) return;  // uniform across the block
  const int64_t i = (t + 1) / m - 1;
  float x = 0.0f;
  if (j < D) {
    Pool1 acc;
    // entry e's positions (c_arr / z_arr: the ring arrays of the values and the logits,
    // B the bias rows); long pooling windows (HCA) in batches of 32 loads, short ones of 8
    auto pool = [&](int64_t e, int c_arr, int z_arr, const float* B) {
      if (m >= 32) pool_positions<32>(acc, ring, m, span, narr, D, j, e, c_arr, z_arr, B);
      else pool_positions<8>(acc, ring, m, span, narr, D, j, e, c_arr, z_arr, B);
    };
    pool(i, 0, overlap ? 2 : 1, Ba);                   // a-branch (CSA arrays 0 = Ca, 2 = Za; HCA 0 = C, 1 = Z)
    if (overlap && i > 0) pool(i - 1, 1, 3, Bb);       // b-branch of the previous entry (arrays 1 = Cb, 3 = Zb)
    x = acc.value();
  }
  x = norm_rope(x, j, D, cv.rope, gain, eps, apply_rope != 0, (double)m * (double)i, base, red);
  store_record(cv, b, i, x, j, red);
}

__global__ void compress_decode_kernel(CacheView cv, int m, int overlap, int in_fmt, const void* new_rows,
                                       const int32_t* pos, float* tail, const float* Ba, const float* Bb,
                                       const float* gain, float eps, int apply_rope, double base) {
  __shared__ float red[16];
  compress_decode_row(cv, m, overlap, in_fmt, new_rows, pos, tail, Ba, Bb, gain, eps, apply_rope, base, blockIdx.x,
                      threadIdx.x, red);
}

__global__ void store_entries_kernel(CacheView cv, int seq, int64_t first, const float* src, const float* gain,
                                     float eps, int apply_rope, double base, int pos_stride) {
  __shared__ float red[16];
  const int D = cv.dim, j = threadIdx.x;
  const int64_t k = blockIdx.x, i = first + k;
  float x = j < D ? src[k * D + j] : 0.0f;
  x = norm_rope(x, j, D, cv.rope, gain, eps, apply_rope != 0, (double)pos_stride * (double)i, base, red);
  store_record(cv, seq, i, x, j, red);
}

// Window append of raw row r (thread j = channel j; every thread of the block takes part).
__device__ __forceinline__ void window_append_row(int D, int R, int in_fmt, int win_fmt, const void* raw,
                                                  const float* gain, const int32_t* pos, const int32_t* seq,
                                                  void* window, int W, int S, float eps, double base, int r, int j,
                                                  float* red, bool row_is_seq = false) {
  const int t = pos ? pos[r] : r;
  const int s = seq ? seq[r] : (row_is_seq ? r : 0);
  float x = j < D ? load_act(raw, in_fmt, (int64_t)r * D + j) : 0.0f;
  x = norm_rope(x, j, D, R, gain, eps, true, (double)t, base, red);
  if (j >= D || t < 0 || s < 0 || s >= S) return;
  int64_t o = ((int64_t)s * W + (t % W)) * D + j;
  if (win_fmt == CA_F32) ((float*)window)[o] = x;
  else ((uint16_t*)window)[o] = f32_to_bf16_bits(x);
}

__global__ void window_append_kernel(int D, int R, int in_fmt, int win_fmt, const void* raw, const float* gain,
                                     const int32_t* pos, const int32_t* seq, void* window, int W, int S, float eps,
                                     double base) {
  __shared__ float red[16];
  window_append_row(D, R, in_fmt, win_fmt, raw, gain, pos, seq, window, W, S, eps, base, blockIdx.x, threadIdx.x,
                    red);
}

// The front of a decode step of a layer in one launch.  For row b (sequence b):
// workgroup (b, 0) appends the new token to its window, (b, 1 + q) runs entry job q's
// compressor step, then (optionally) ceil(n_heads / waves) workgroups prepare the
// row's attention queries (one wavefront per head), and one clears the row's long
// top-k state.  Each workgroup does exactly what the workgroup of the separate
// launch does, so the results are the same bit for bit.
__global__ void decode_front_kernel(DecodeWindowJob wj, DecodeEntryJob e0, DecodeEntryJob e1, int n_jobs,
                                    AttendArgs qa, uint32_t* zero, int zero_words, const int32_t* pos) {
  __shared__ float red[16];
  const int b = blockIdx.x, j = threadIdx.x, y = blockIdx.y;
  if (y == 0) {
    window_append_row(wj.D, wj.R, wj.in_fmt, wj.win_fmt, wj.raw, wj.gain, pos, nullptr, wj.window, wj.W, wj.S,
                      wj.eps, wj.base, b, j, red, true);
    return;
  }
  if (y <= n_jobs) {
    const DecodeEntryJob& e = y == 1 ? e0 : e1;
    compress_decode_row(e.cv, e.m, e.overlap, e.in_fmt, e.new_rows, pos, e.tail, e.Ba, e.Bb, e.gain, e.eps,
                        e.apply_rope, e.base, b, j, red);
    return;
  }
  const int hpb = blockDim.x >> 6;                     // heads per workgroup
  const int n_q = qa.q_prep != nullptr ? (qa.n_heads + hpb - 1) / hpb : 0;
  if (y <= n_jobs + n_q) {
    const int h = (y - 1 - n_jobs) * hpb + (j >> 6);
    if (h < qa.n_heads) qprep_head(qa, b, h, j & 63);
    return;
  }
  for (int i = j; i < zero_words; i += blockDim.x) zero[(int64_t)b * zero_words + i] = 0u;
}

// ----------------------------------------------------------------- launchers
static int block_for(int D) { return (D + 63) / 64 * 64; }

hipError_t launch_compress_prefill(const CacheView& cv, int seq, const ca_compress_params& p, const void* Ca,
                                   const void* Za, const void* Cb, const void* Zb, const float* Ba,
                                   const float* Bb, const float* gain, int64_t L, int64_t t0, hipStream_t st) {
  const int64_t i0 = compress_first_entry(p.ratio, p.overlap, t0), i1 = (t0 + L) / p.ratio;
  if (i1 <= i0) return hipSuccess;
  hipLaunchKernelGGL(compress_prefill_kernel, dim3((unsigned)(i1 - i0)), dim3(block_for(cv.dim)), 0, st, cv, seq,
                     p.ratio, p.overlap, p.in_format, Ca, Za, Cb, Zb, Ba, Bb, p.apply_norm ? gain : nullptr, p.eps,
                     p.apply_rope, p.rope_base, i0, t0);
  return hipGetLastError();
}

hipError_t launch_compress_decode(const CacheView& cv, const ca_compress_params& p, const void* new_rows,
                                  const int32_t* pos, int B, float* tail, const float* Ba, const float* Bb,
                                  const float* gain, hipStream_t st) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_decode_kernel, dim3(B), dim3(block_for(cv.dim)), 0, st, cv, p.ratio, p.overlap,
                     p.in_format, new_rows, pos, tail, Ba, Bb, p.apply_norm ? gain : nullptr, p.eps, p.apply_rope,
                     p.rope_base);
  return hipGetLastError();
}

hipError_t launch_store_entries(const CacheView& cv, int seq, int64_t first, int64_t n, const float* src,
                                const float* gain, float eps, int apply_rope, double base, int pos_stride,
                                hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(store_entries_kernel, dim3((unsigned)n), dim3(block_for(cv.dim)), 0, st, cv, seq, first, src,
                     gain, eps, apply_rope, base, pos_stride);
  return hipGetLastError();
}

hipError_t launch_decode_front(const DecodeWindowJob& wj, const DecodeEntryJob* jobs, int n_jobs,
                               const int32_t* pos, int B, const AttendArgs* qa, uint32_t* zero, int zero_words,
                               hipStream_t st) {
  if (B == 0) return hipSuccess;
  int threads = block_for(wj.D);
  for (int q = 0; q < n_jobs; ++q) threads = block_for(jobs[q].cv.dim) > threads ? block_for(jobs[q].cv.dim) : threads;
  AttendArgs a{};
  if (qa != nullptr && qa->q_prep != nullptr) a = *qa;
  const int n_q = a.q_prep != nullptr ? (a.n_heads + threads / 64 - 1) / (threads / 64) : 0;
  const int n_zero = zero != nullptr && zero_words > 0 ? 1 : 0;
  hipLaunchKernelGGL(decode_front_kernel, dim3(B, 1 + n_jobs + n_q + n_zero), dim3(threads), 0, st, wj, jobs[0],
                     n_jobs > 1 ? jobs[1] : jobs[0], n_jobs, a, n_zero ? zero : nullptr, n_zero ? zero_words : 0, pos);
  return hipGetLastError();
}

hipError_t launch_decode_append(const DecodeWindowJob& wj, const DecodeEntryJob* jobs, int n_jobs,
                                const int32_t* pos, int B, hipStream_t st) {
  return launch_decode_front(wj, jobs, n_jobs, pos, B, nullptr, nullptr, 0, st);
}

hipError_t launch_window_append(const ca_window_params& p, const void* raw, const float* gain, const int32_t* pos,
                                const int32_t* seq, int T, void* window, int W, int S, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(window_append_kernel, dim3(T), dim3(block_for(p.dim)), 0, st, p.dim, p.rope_dim, p.in_format,
                     p.win_format, raw, gain, pos, seq, window, W, S, p.eps, p.rope_base);
  return hipGetLastError();
}

}  // namespace ca
