// Shared device helpers of the CSA / HCA kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csahca.h"

namespace ca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> OCP e4m3fn code, round to nearest even, saturating to +-448.
// Normal results are rounded on the float bit pattern (carry into the
// exponent is automatic); results below 2^-6 land on the 2^-9 subnormal grid.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t s = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return s | 0x7Eu;            // |x| >= 448 (or NaN/inf): saturate
  if (a < 0x3C800000u) {                              // |x| < 2^-6
    float q = rintf(__uint_as_float(a) * 512.0f);     // exact scaling, RNE
    return s | (uint32_t)q;                           // 0..8 (8 is the smallest normal)
  }
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);       // RNE at mantissa bit 20 (3 bits kept)
  int E = (int)((r >> 23) & 0xFFu) - 127 + 7;
  uint32_t mant = (r >> 20) & 7u;
  if (E > 15 || (E == 15 && mant == 7)) return s | 0x7Eu;
  return s | ((uint32_t)E << 3) | mant;
}

// Smallest e with amax <= 448 * 2^e (0 when amax == 0); exact.
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ea;
  float f = frexpf(amax, &ea);          // amax = f * 2^ea, f in [0.5, 1); 448 = 0.875 * 2^9
  return f <= 0.875f ? ea - 9 : ea - 8;
}

// float -> OCP e2m1 (FP4) code: nearest of the magnitudes 0, .5, 1, 1.5, 2, 3,
// 4, 6 by comparison with the midpoints between them, a midpoint going to the
// code with mantissa bit 0; saturates to +-6; magnitude 0 is encoded +0.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return (x < 0.0f && c != 0u) ? (c | 8u) : c;
}

// e2m1 code -> float, exact.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float v = e == 0u ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
  return (c & 8u) ? -v : v;
}

// Smallest e with amax <= 6 * 2^e (0 when amax == 0), clamped to the E8M0
// range [-127, 127]; exact.
__device__ __forceinline__ int fp4_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int ea;
  const float f = frexpf(amax, &ea);    // amax = f * 2^ea, f in [0.5, 1); 6 = 0.75 * 2^3
  const int e = f <= 0.75f ? ea - 3 : ea - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two e4m3 codes (bytes 0,1 or, with HI, 2,3 of `word`) -> two floats, exact.
template <bool HI = false>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
}

// Two e4m3 codes scaled by a power of two -> two bf16 (exact for the ranges used here).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16_scaled(uint32_t word, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)word, scale, HI);
}

// ----------------------------------------------------------------- records
__host__ __device__ __forceinline__ int64_t record_stride(int fmt, int D, int R) {
  switch (fmt) {
    case CA_F32: return 4 * (int64_t)D;
    case CA_BF16: return 2 * (int64_t)D;
    case CA_FP8MIX: {
      int64_t raw = (int64_t)(D - R) + 2 * R + (D - R) / 64;
      return (raw + 127) / 128 * 128;
    }
    case CA_E4M3: return D;
    case CA_FP4: return D / 2;
  }
  return -1;
}

__host__ __device__ __forceinline__ int64_t page_bytes(int fmt, int D, int R, int P) {
  if (fmt == CA_E4M3) return (int64_t)P * D + 4 * (int64_t)P;
  if (fmt == CA_FP4) return (int64_t)P * (D / 2) + (int64_t)P * (D / 32);
  return (int64_t)P * record_stride(fmt, D, R);
}

// First entry a prefill whose rows start at position t0 emits: the first whose
// pooling window (m rows, plus the m rows before them when overlapping, except
// for entry 0) lies at or after t0.
__host__ __device__ __forceinline__ int64_t compress_first_entry(int m, int overlap, int64_t t0) {
  if (t0 <= 0) return 0;
  const int64_t a = (t0 + m - 1) / m;                   // first block starting at or after t0
  return overlap ? a + 1 : a;
}

// Device view of a paged pool.
struct CacheView {
  uint8_t* pool;
  const int32_t* page_table;
  int64_t n_pages;
  int64_t page_bytes;
  int64_t stride;
  int32_t max_pages;
  int32_t page_shift;  // log2(page_size)
  int32_t fmt, dim, rope;

  // Page base of entry i of sequence s, or nullptr if its page is missing.
  __device__ __forceinline__ uint8_t* page_of(int s, int64_t i) const {
    int64_t pi = i >> page_shift;
    if (i < 0 || pi >= max_pages) return nullptr;
    int32_t pg = page_table[(int64_t)s * max_pages + pi];
    if (pg < 0 || pg >= n_pages) return nullptr;
    return pool + (int64_t)pg * page_bytes;
  }
  __device__ __forceinline__ int slot_of(int64_t i) const { return (int)(i & ((1 << page_shift) - 1)); }
  __device__ __forceinline__ uint8_t* entry(int s, int64_t i) const {
    uint8_t* p = page_of(s, i);
    return p ? p + slot_of(i) * stride : nullptr;
  }
};

// ----------------------------------------------------------------- rope
// Angle of rotary pair p at position pos, in double precision (positions reach
// 2^20, where a float product would lose ~0.06 rad).
__device__ __forceinline__ void rope_sincos(double pos, int p, int R, double base, float* s, float* c) {
  double theta = pow(base, -2.0 * (double)p / (double)R);
  double sn, cs;
  sincos(pos * theta, &sn, &cs);
  *s = (float)sn;
  *c = (float)cs;
}

// ----------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float load_act(const void* p, int fmt, int64_t i) {
  return fmt == CA_F32 ? ((const float*)p)[i] : bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

}  // namespace ca
