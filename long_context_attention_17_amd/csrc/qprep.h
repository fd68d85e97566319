// Query preparation of split (decode) rows for the MFMA attention path, shared by
// attend_qprep_kernel and the fused decode front kernel: RMSNorm with gain, RoPE at
// the row's position, logit scale * log2(e) -- once per (row, head) instead of once
// per split (dsv4 book Ch.7 "Query and KV RMSNorm", "Partial RoPE and output
// de-rotation").  The row is stored in bf16 without the norm's factor 1 / rms
// (x * gain * scale, rotated), which goes to q_inv and scales the head's logits: the
// same rounding as the attention kernel's own transform of raw queries.  One
// wavefront per (row, head), lane l holding channels 8l .. 8l+7.
#pragma once
#include "common.h"
#include "kernels.h"

namespace ca {

__device__ __forceinline__ void qprep_head(const AttendArgs& a, int r, int h, int lane) {
  constexpr int kD = 512, kR = 64, CC = kD - kR;
  const int t = a.pos ? a.pos[r] : a.t0 + r;
  const int64_t off = ((int64_t)r * a.n_heads + h) * kD + 8 * lane;
  const u32x4 w = *(const u32x4*)((const uint16_t*)a.q + off);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (lane == 0) a.q_inv[(int64_t)r * a.n_heads + h] = 1.0f / sqrtf(ss / (float)kD + a.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= a.q_gain[8 * lane + e] * a.scale_log2;
  if (8 * lane >= CC) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int p = (8 * lane + e - CC) >> 1;
      double th = 1.0, bp = a.rope_step;
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        th = ((p >> k) & 1) ? th * bp : th;
        bp *= bp;
      }
      const double rev = (double)t * th * 0.15915494309189535;   // 1 / (2 pi)
      const float fr = (float)(rev - floor(rev));
      const float c = __builtin_amdgcn_cosf(fr), sn = __builtin_amdgcn_sinf(fr);
      const float x0 = x[e], x1 = x[e + 1];
      x[e] = x0 * c - x1 * sn;
      x[e + 1] = x0 * sn + x1 * c;
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x[2 * e], (__bf16)x[2 * e + 1]});
  *(u32x4*)(a.q_prep + off) = o;
}

}  // namespace ca
