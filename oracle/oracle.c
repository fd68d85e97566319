/*
 * CPU ORACLE for compressed sparse attention (CSA) and heavily compressed
 * attention (HCA).  TEST INFRASTRUCTURE ONLY: it is read by tests/, by the
 * smoke check and by the CPU-baseline leg of bench.py, and by nothing in the
 * product path.  It shares no code, header or table with the HIP library.
 *
 * Everything is computed in double precision with plain loops, in the order
 * the definitions are written, so a reader can check it against the source
 * pages by eye.  The only roundings are the storage formats (bf16, OCP e4m3
 * with power-of-two scales, OCP e2m1 with E8M0 block scales) that the method
 * itself stores its cache in.
 *
 * Sources (all on the "DeepSeek-V4" technical-report walkthrough book, page
 * slop-6tp.pages.dev/papers-html-argon/dsv4.html, hereafter "dsv4 book"):
 *   - Ch.5 "How CSA Compresses Memory": four compression projections,
 *     coordinate-wise softmax pooling, receptive field vs stride (first-block
 *     rule, floor(N/m) completed entries), causal availability.
 *   - Ch.6 "How CSA Selects and Reads Memory": lightning indexer score
 *     (ReLU, per-head combiner weights), top-k over blocks s < floor(t/m),
 *     shared key-value MQA.
 *   - Ch.7 "HCA, Local Attention, and Position": 128:1 disjoint compressor,
 *     dense attention over i < floor(t/m'), the uncompressed sliding window in
 *     one unified softmax, query/KV RMSNorm, partial RoPE on the last
 *     coordinates with output de-rotation by R_{-t}, learned attention sinks.
 *   - Ch.2 "What an attention head computes": logits scaled by the head
 *     dimension c (read as 1/sqrt(c)); "Normalization and rotary position
 *     embeddings": RMSNorm with learned gain g and epsilon.
 *   - Ch.8 "A Cost Model for Long Context", "V4 compressed-entry payload":
 *     448 content channels in FP8 plus 64 rotary channels in BF16.
 * Points the pages leave open are fixed by the readings listed in the design
 * notes (eligibility s < floor(t/m), window = last n_win positions including
 * t with no de-duplication, entry RoPE position m*i, RoPE pairs (2p,2p+1)
 * with theta_p = base^(-2p/R), scale 1/sqrt(D), e4m3 with one power-of-two
 * exponent per 64-channel tile).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_E4M3_MAX 448.0

/* ------------------------------------------------------------------ */
/* Storage number formats                                              */
/* ------------------------------------------------------------------ */

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, 0x7F / 0xFF are NaN, largest finite 448, subnormals
 * m * 2^-9. */
double orc_e4m3_decode(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* Round-to-nearest-even to E4M3, saturating to +-448 (satfinite). */
uint8_t orc_e4m3_encode(double x) {
  uint8_t s = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7F;
  if (a >= ORC_E4M3_MAX) return s | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal grid of spacing 2^-9 (q == 8 is the smallest normal) */
    double q = nearbyint(ldexp(a, 9));
    return s | (uint8_t)q;
  }
  int e;
  double f = frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
  double q = nearbyint(f * 16.0);   /* 4 significant bits: q in [8, 16] */
  if (q == 16.0) { q = 8.0; e += 1; }
  int E = (e - 1) + 7;              /* value = (q/8) * 2^(e-1) */
  int mant = (int)q - 8;
  if (E > 15 || (E == 15 && mant == 7)) return s | 0x7E;
  return s | (uint8_t)((E << 3) | mant);
}

double orc_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round-to-nearest-even of a double to bfloat16 (8 significant bits),
 * computed directly from the double (no intermediate float rounding). */
uint16_t orc_bf16_encode(double x) {
  if (isnan(x)) return 0x7FC0;
  double r;
  double a = fabs(x);
  if (a == 0) {
    r = x;
  } else if (a < ldexp(1.0, -126)) {
    r = ldexp(nearbyint(ldexp(x, 133)), -133);
  } else {
    int e;
    double f = frexp(x, &e);                  /* |f| in [0.5, 1) */
    r = ldexp(nearbyint(f * 256.0), e - 8);   /* 8 significant bits, RNE */
  }
  float rf = (float)r;                         /* exact: r has <= 8 bits */
  uint32_t u;
  memcpy(&u, &rf, 4);
  return (uint16_t)(u >> 16);
}

/* Smallest integer e with amax <= 448 * 2^e, i.e. e = ceil(log2(amax/448));
 * 0 when amax == 0.  Computed with exact comparisons. */
int orc_pow2_exponent(double amax) {
  if (!(amax > 0)) return 0;
  int e = (int)ceil(log2(amax / ORC_E4M3_MAX));
  while (amax > ldexp(ORC_E4M3_MAX, e)) e++;
  while (amax <= ldexp(ORC_E4M3_MAX, e - 1)) e--;
  return e;
}

void orc_encode_bf16_array(int64_t n, const double* x, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode(x[i]);
}
void orc_decode_bf16_array(int64_t n, const uint16_t* x, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(x[i]);
}
void orc_decode_e4m3_array(int64_t n, const uint8_t* x, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(x[i]);
}

/* Quantize rows of length c to e4m3 with one power-of-two scale per row
 * (used for indexer queries and indexer keys). */
void orc_quantize_rows_e4m3(int64_t n, int c, const double* x, uint8_t* codes, int32_t* exps) {
  for (int64_t i = 0; i < n; ++i) {
    double amax = 0;
    for (int j = 0; j < c; ++j) amax = fmax(amax, fabs(x[i * c + j]));
    int e = orc_pow2_exponent(amax);
    exps[i] = e;
    for (int j = 0; j < c; ++j) codes[i * c + j] = orc_e4m3_encode(ldexp(x[i * c + j], -e));
  }
}

/* OCP FP4 E2M1 (MX element format, the indexer-key precision of the
 * dsv4 book Ch.6 "The lightning indexer" and Ch.8 "Quantization scales and
 * bounded tail buffers"): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
 * bit, no infinities or NaN.  Code bits: [3] sign, [2:1] exponent, [0]
 * mantissa; exponent 0 is subnormal (0 or 0.5). */
double orc_e2m1_decode(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Nearest E2M1 value by exhaustive search over the 8 magnitudes, ties to the
 * even code (mantissa bit 0); beyond 6 the nearest is 6 (saturation).  A
 * result of magnitude 0 is encoded +0. */
uint8_t orc_e2m1_encode(double x) {
  double a = fabs(x);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(a - orc_e2m1_decode((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)((x < 0 && best != 0) ? (best | 8) : best);
}

/* Block exponent of an FP4 block: the smallest e with amax <= 6 * 2^e (so no
 * element saturates), 0 when amax == 0, clamped to the E8M0 range
 * [-127, 127].  Stored as the E8M0 byte e + 127 (value 2^e). */
int orc_fp4_block_exponent(double amax) {
  if (!(amax > 0)) return 0;
  int e = (int)ceil(log2(amax / 6.0));
  while (amax > ldexp(6.0, e)) e++;
  while (amax <= ldexp(6.0, e - 1)) e--;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

void orc_decode_e2m1_array(int64_t n, const uint8_t* x, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_decode(x[i]);
}

/* ------------------------------------------------------------------ */
/* Record and page layout of the compressed caches                     */
/* ------------------------------------------------------------------ */
/* fmt 0: fp32 record, D floats.
 * fmt 1: bf16 record, D bf16 (RNE).
 * fmt 2: mixed record (dsv4 book Ch.8, V4 compressed-entry payload): the first
 *        D-R channels as e4m3 codes, one signed int8 power-of-two exponent per
 *        64-channel tile of them, and the last R (rotary) channels as bf16.
 *        Bytes: [codes D-R][bf16 2R][exponents (D-R)/64][zero pad] with the
 *        record stride rounded up to 128 bytes (640 B for D=512, R=64).
 * fmt 3: indexer key page, structure of arrays: [P*D e4m3 codes][P fp32 scales].
 * fmt 4: indexer key page in FP4 (dsv4 book Ch.8: 0.5 byte per scalar plus a
 *        1-byte scale per 32 elements): [P*D/2 bytes of E2M1 codes, channel
 *        2k in the low nibble of byte k, channel 2k+1 in the high nibble]
 *        [P*D/32 E8M0 block-scale bytes, block b of slot i at i*D/32 + b].
 * A page holds P entries; entry i of a sequence is in page
 * page_table_row[i / P] at slot i % P. */

int64_t orc_record_stride(int fmt, int D, int R) {
  switch (fmt) {
    case 0: return 4 * (int64_t)D;
    case 1: return 2 * (int64_t)D;
    case 2: {
      int64_t raw = (D - R) + 2 * R + (D - R) / 64;
      return (raw + 127) / 128 * 128;
    }
    case 3: return D;  /* codes only; scales live at the end of the page */
    case 4: return D / 2;
  }
  return -1;
}

int64_t orc_page_bytes(int fmt, int D, int R, int P) {
  if (fmt == 3) return (int64_t)P * D + 4 * (int64_t)P;
  if (fmt == 4) return (int64_t)P * (D / 2) + (int64_t)P * (D / 32);
  return (int64_t)P * orc_record_stride(fmt, D, R);
}

static uint8_t* entry_ptr(int fmt, int D, int R, int P, uint8_t* pool, const int32_t* pt_row, int64_t i) {
  int64_t page = pt_row[i / P];
  int64_t slot = i % P;
  return pool + page * orc_page_bytes(fmt, D, R, P) + slot * orc_record_stride(fmt, D, R);
}

/* Encode one entry x[D] (already normalized / rotated) into the pool. */
void orc_store_entry(int fmt, int D, int R, int P, uint8_t* pool, const int32_t* pt_row, int64_t i, const double* x) {
  uint8_t* p = entry_ptr(fmt, D, R, P, pool, pt_row, i);
  if (fmt == 0) {
    for (int j = 0; j < D; ++j) { float f = (float)x[j]; memcpy(p + 4 * j, &f, 4); }
  } else if (fmt == 1) {
    for (int j = 0; j < D; ++j) { uint16_t b = orc_bf16_encode(x[j]); memcpy(p + 2 * j, &b, 2); }
  } else if (fmt == 2) {
    int C = D - R, ntile = C / 64;
    memset(p, 0, (size_t)orc_record_stride(fmt, D, R));
    for (int t = 0; t < ntile; ++t) {
      double amax = 0;
      for (int j = 0; j < 64; ++j) amax = fmax(amax, fabs(x[64 * t + j]));
      int e = orc_pow2_exponent(amax);
      p[C + 2 * R + t] = (uint8_t)(int8_t)e;
      for (int j = 0; j < 64; ++j) p[64 * t + j] = orc_e4m3_encode(ldexp(x[64 * t + j], -e));
    }
    for (int j = 0; j < R; ++j) { uint16_t b = orc_bf16_encode(x[C + j]); memcpy(p + C + 2 * j, &b, 2); }
  } else if (fmt == 3) {
    double amax = 0;
    for (int j = 0; j < D; ++j) amax = fmax(amax, fabs(x[j]));
    int e = orc_pow2_exponent(amax);
    for (int j = 0; j < D; ++j) p[j] = orc_e4m3_encode(ldexp(x[j], -e));
    int64_t page = pt_row[i / P];
    uint8_t* sc = pool + page * orc_page_bytes(fmt, D, R, P) + (int64_t)P * D + 4 * (i % P);
    float f = (float)ldexp(1.0, e);
    memcpy(sc, &f, 4);
  } else if (fmt == 4) {
    int64_t page = pt_row[i / P];
    uint8_t* sc = pool + page * orc_page_bytes(fmt, D, R, P) + (int64_t)P * (D / 2) + (i % P) * (D / 32);
    for (int b = 0; b < D / 32; ++b) {
      double amax = 0;
      for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs(x[32 * b + j]));
      int e = orc_fp4_block_exponent(amax);
      sc[b] = (uint8_t)(e + 127);
      for (int j = 0; j < 32; j += 2) {
        uint8_t lo = orc_e2m1_encode(ldexp(x[32 * b + j], -e));
        uint8_t hi = orc_e2m1_encode(ldexp(x[32 * b + j + 1], -e));
        p[(32 * b + j) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

/* Decode one entry from the pool into x[D] (exact values of the stored format). */
void orc_load_entry(int fmt, int D, int R, int P, const uint8_t* pool, const int32_t* pt_row, int64_t i, double* x) {
  const uint8_t* p = entry_ptr(fmt, D, R, P, (uint8_t*)pool, pt_row, i);
  if (fmt == 0) {
    for (int j = 0; j < D; ++j) { float f; memcpy(&f, p + 4 * j, 4); x[j] = f; }
  } else if (fmt == 1) {
    for (int j = 0; j < D; ++j) { uint16_t b; memcpy(&b, p + 2 * j, 2); x[j] = orc_bf16_decode(b); }
  } else if (fmt == 2) {
    int C = D - R, ntile = C / 64;
    for (int t = 0; t < ntile; ++t) {
      int e = (int8_t)p[C + 2 * R + t];
      for (int j = 0; j < 64; ++j) x[64 * t + j] = ldexp(orc_e4m3_decode(p[64 * t + j]), e);
    }
    for (int j = 0; j < R; ++j) { uint16_t b; memcpy(&b, p + C + 2 * j, 2); x[C + j] = orc_bf16_decode(b); }
  } else if (fmt == 3) {
    int64_t page = pt_row[i / P];
    const uint8_t* sc = pool + page * orc_page_bytes(fmt, D, R, P) + (int64_t)P * D + 4 * (i % P);
    float f;
    memcpy(&f, sc, 4);
    for (int j = 0; j < D; ++j) x[j] = orc_e4m3_decode(p[j]) * (double)f;
  } else if (fmt == 4) {
    int64_t page = pt_row[i / P];
    const uint8_t* sc = pool + page * orc_page_bytes(fmt, D, R, P) + (int64_t)P * (D / 2) + (i % P) * (D / 32);
    for (int j = 0; j < D; ++j) {
      uint8_t code = (j & 1) ? (p[j / 2] >> 4) : (p[j / 2] & 15);
      x[j] = ldexp(orc_e2m1_decode(code), (int)sc[j / 32] - 127);
    }
  }
}

/* ------------------------------------------------------------------ */
/* RMSNorm and partial RoPE                                            */
/* ------------------------------------------------------------------ */

/* dsv4 book Ch.2 "Normalization and rotary position embeddings" and Ch.7
 * "Query and KV RMSNorm": y = x / sqrt(mean(x^2) + eps) * g. */
void orc_rmsnorm(int n, const double* x, const double* g, double eps, double* y) {
  double ss = 0;
  for (int j = 0; j < n; ++j) ss += x[j] * x[j];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int j = 0; j < n; ++j) y[j] = x[j] * inv * g[j];
}

/* dsv4 book Ch.7 "Partial RoPE and output de-rotation": the last R of D
 * coordinates are rotated pairwise, pair p = (D-R+2p, D-R+2p+1), by the angle
 * pos * theta_p with theta_p = base^(-2p/R).  sign=-1 applies R_{-pos} = R_pos^T. */
void orc_rope(int D, int R, double base, double pos, int sign, double* x) {
  for (int p = 0; p < R / 2; ++p) {
    double theta = pow(base, -2.0 * p / R);
    double ang = sign * pos * theta;
    double c = cos(ang), s = sin(ang);
    double a = x[D - R + 2 * p], b = x[D - R + 2 * p + 1];
    x[D - R + 2 * p] = a * c - b * s;
    x[D - R + 2 * p + 1] = a * s + b * c;
  }
}

/* ------------------------------------------------------------------ */
/* Compressors                                                          */
/* ------------------------------------------------------------------ */

/* One compressed entry from its source token rows.
 * overlap = 1 (CSA, dsv4 book Ch.5 "Coordinate-wise softmax pooling"): for each
 *   coordinate r, softmax over the 2m logits Za[j,r] + Ba[j,r] (current block,
 *   j < m) and Zb[j,r] + Bb[j,r] (previous block), then the weighted sum of the
 *   matching Ca / Cb contents.  has_prev = 0 is the first-block rule (Ch.5
 *   "Receptive field versus compression stride"): b-branch logits are -inf and
 *   its contents zero, so the softmax runs over the current block only.
 * overlap = 0 (HCA, Ch.7 "HCA's 128:1 non-overlapping compressor"): softmax
 *   over the m rows of Za + Ba, weighted sum of Ca.
 * Rows are [m, c] row-major; out[c]. */
void orc_compress_entry(int c, int m, int overlap, int has_prev,
                        const double* Ca, const double* Za, const double* Cb, const double* Zb,
                        const double* Ba, const double* Bb, double* out) {
  int use_b = overlap && has_prev;
  for (int r = 0; r < c; ++r) {
    double mx = -INFINITY;
    for (int j = 0; j < m; ++j) mx = fmax(mx, Za[j * c + r] + Ba[j * c + r]);
    if (use_b)
      for (int j = 0; j < m; ++j) mx = fmax(mx, Zb[j * c + r] + Bb[j * c + r]);
    double den = 0, num = 0;
    for (int j = 0; j < m; ++j) {
      double w = exp(Za[j * c + r] + Ba[j * c + r] - mx);
      den += w;
      num += w * Ca[j * c + r];
    }
    if (use_b)
      for (int j = 0; j < m; ++j) {
        double w = exp(Zb[j * c + r] + Bb[j * c + r] - mx);
        den += w;
        num += w * Cb[j * c + r];
      }
    out[r] = num / den;
  }
}

/* All completed entries of a sequence of L token rows: floor(L/m) of them
 * (the trailing partial block is not emitted).  Ca..Zb are [L, c]. */
int64_t orc_compress(int64_t L, int c, int m, int overlap,
                     const double* Ca, const double* Za, const double* Cb, const double* Zb,
                     const double* Ba, const double* Bb, double* out) {
  int64_t n = L / m;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int has_prev = i > 0;
    const double* cb = has_prev && overlap ? Cb + (i - 1) * m * (int64_t)c : NULL;
    const double* zb = has_prev && overlap ? Zb + (i - 1) * m * (int64_t)c : NULL;
    orc_compress_entry(c, m, overlap, has_prev, Ca + i * m * (int64_t)c, Za + i * m * (int64_t)c, cb, zb, Ba, Bb,
                       out + i * (int64_t)c);
  }
  return n;
}

/* Entry epilogue and store: for entries first..first+n-1 of one sequence,
 * optional RMSNorm (gain g, eps), optional RoPE at position ratio*i, then
 * encode into the pool in format fmt. */
void orc_finish_store(int fmt, int D, int R, int P, uint8_t* pool, const int32_t* pt_row,
                      int64_t first, int64_t n, const double* x, const double* g, double eps,
                      double base, int ratio, int apply_norm, int apply_rope) {
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(static)
    for (int64_t k = 0; k < n; ++k) {
      int64_t i = first + k;
      if (apply_norm) orc_rmsnorm(D, x + k * (int64_t)D, g, eps, y);
      else memcpy(y, x + k * (int64_t)D, sizeof(double) * D);
      if (apply_rope && R > 0) orc_rope(D, R, base, (double)ratio * (double)i, 1, y);
      orc_store_entry(fmt, D, R, P, pool, pt_row, i, y);
    }
    free(y);
  }
}

/* Decode many entries (oracle view of a pool). */
void orc_load_entries(int fmt, int D, int R, int P, const uint8_t* pool, const int32_t* pt_row,
                      int64_t first, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) orc_load_entry(fmt, D, R, P, pool, pt_row, first + k, out + k * (int64_t)D);
}

/* Window token: RMSNorm (gain g) then RoPE at the token's own position. */
void orc_window_prep(int64_t n, int D, int R, double base, double eps, const double* raw, const double* g,
                     const int64_t* pos, double* out) {
  for (int64_t k = 0; k < n; ++k) {
    orc_rmsnorm(D, raw + k * D, g, eps, out + k * D);
    if (R > 0) orc_rope(D, R, base, (double)pos[k], 1, out + k * D);
  }
}

/* ------------------------------------------------------------------ */
/* Lightning indexer and top-k                                          */
/* ------------------------------------------------------------------ */

/* dsv4 book Ch.6 "The lightning indexer": for query row r at position t and
 * every block s < floor(t/m) (Ch.5 "Causal availability"),
 *   I[t,s] = sum_h w[t,h] * ReLU( qI[t,h,:] . K[s,:] ).
 * qI holds the (dequantized) indexer query values [n_rows, nI, cI]; keys are
 * read from the indexer pool (fmt 0, 3 or 4).  Scores beyond the eligible count
 * are left untouched.  n_elig[r] = min(floor(t/m), n_avail[seq]). */
int orc_index_scores(int64_t n_rows, int nI, int cI, int m, const double* qI, const double* w,
                     const int64_t* pos, const int32_t* seq, int idx_fmt, int P, const uint8_t* pool,
                     const int32_t* page_table, int max_pages, const int64_t* n_avail,
                     int64_t row_stride, double* scores, int64_t* n_elig) {
  int bad = 0;
  /* rows one after another; the keys of a row are shared out among the threads
   * (each score is computed by one thread, in the order written above) */
  for (int64_t r = 0; r < n_rows; ++r) {
    int s_id = seq ? seq[r] : 0;
    int64_t ne = pos[r] / m;
    if (ne > n_avail[s_id]) {
      bad = 1;
      ne = n_avail[s_id];
    }
    n_elig[r] = ne;
    const int32_t* pt = page_table + (int64_t)s_id * max_pages;
#pragma omp parallel
    {
      double* key = (double*)malloc(sizeof(double) * cI);
#pragma omp for schedule(static, 256)
      for (int64_t s = 0; s < ne; ++s) {
        orc_load_entry(idx_fmt, cI, 0, P, pool, pt, s, key);
        double acc = 0;
        for (int h = 0; h < nI; ++h) {
          const double* q = qI + (r * nI + h) * (int64_t)cI;
          double dot = 0;
          for (int j = 0; j < cI; ++j) dot += q[j] * key[j];
          acc += w[r * nI + h] * (dot > 0 ? dot : 0);
        }
        scores[r * row_stride + s] = acc;
      }
      free(key);
    }
  }
  return bad ? -1 : 0;
}

typedef struct { double v; int64_t i; } orc_pair;
static int pair_cmp(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  if (x->v > y->v) return -1;     /* larger score first */
  if (x->v < y->v) return 1;
  return (x->i < y->i) ? -1 : (x->i > y->i);  /* tie: lower index first */
}
static int idx_cmp(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* dsv4 book Ch.6 "Top-k selection and asymptotic scaling": keep the
 * min(k, n_elig) blocks with the largest score; ties go to the lower block
 * index; the kept indices are written in ascending order and the rest of the
 * row is padded with -1. */
void orc_topk(int64_t n_rows, int64_t row_stride, const double* scores, const int64_t* n_elig, int k,
              int32_t* idx, int32_t* cnt) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t n = n_elig[r];
    orc_pair* a = (orc_pair*)malloc(sizeof(orc_pair) * (n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) { a[s].v = scores[r * row_stride + s]; a[s].i = s; }
    qsort(a, (size_t)n, sizeof(orc_pair), pair_cmp);
    int64_t c = n < k ? n : k;
    for (int64_t j = 0; j < c; ++j) idx[r * k + j] = (int32_t)a[j].i;
    qsort(idx + r * k, (size_t)c, sizeof(int32_t), idx_cmp);
    for (int64_t j = c; j < k; ++j) idx[r * k + j] = -1;
    cnt[r] = (int32_t)c;
    free(a);
  }
}

/* ------------------------------------------------------------------ */
/* Core attention                                                       */
/* ------------------------------------------------------------------ */

/* One query row (position t) of CSA or HCA core attention
 * (dsv4 book Ch.6 "Shared key-value MQA", Ch.7 "Dense attention over heavily
 * compressed history", "The 128-token uncompressed sliding window", "Query
 * and KV RMSNorm", "Partial RoPE and output de-rotation", "Learned attention
 * sinks"):
 *   q^_h  = RoPE_t(RMSNorm(q_h; gq))
 *   X     = {compressed entries of the row} U {window tokens max(0,t-n_win+1)..t}
 *   z_x   = scale * q^_h . x
 *   o_h   = sum_x e^{z_x} x / (sum_x e^{z_x} + e^{sink_h})
 *   o_h[D-R:] <- R_{-t} o_h[D-R:]
 * mode 0 (CSA): the entries are idx[r, 0..cnt[r]).
 * mode 1 (HCA): the entries are 0..floor(t/ratio)-1.
 * Window tokens are read as stored (already normalized and rotated) from
 * win[seq, pos mod W, :] in win_fmt 0 (fp32) or 1 (bf16).
 * Returns -1 when a needed entry is missing from the cache. */
int orc_attend(int64_t n_rows, int nh, int D, int R, double base, double scale, double eps,
               const double* q, const double* gq, const int64_t* pos, const int32_t* seq,
               int kv_fmt, int P, const uint8_t* kv_pool, const int32_t* page_table, int max_pages,
               const int64_t* n_avail, int mode, int ratio, const int32_t* idx, const int32_t* cnt, int k,
               int n_win, int win_fmt, const void* win, int W, const double* sink,
               double* out, double* lse) {
  int bad = 0;
  int64_t cap = 0;
  double* X = NULL;
  /* rows one after another: a row's items are decoded once (shared out among the
   * threads), then its heads are shared out among the threads, each head computed
   * by one thread in the order written here */
  for (int64_t r = 0; r < n_rows; ++r) {
    int s_id = seq ? seq[r] : 0;
    int64_t t = pos[r];
    const int32_t* pt = page_table + (int64_t)s_id * max_pages;
    int64_t ne = mode == 0 ? cnt[r] : t / ratio;
    int64_t w0 = t - n_win + 1 < 0 ? 0 : t - n_win + 1;
    int64_t nw = t - w0 + 1;
    int64_t nx = ne + nw;
    if (nx > cap) {
      cap = nx;
      X = (double*)realloc(X, sizeof(double) * D * cap);
    }
    int ok = 1;
#pragma omp parallel for schedule(static, 64)
    for (int64_t j = 0; j < ne; ++j) {
      int64_t e = mode == 0 ? idx[r * (int64_t)k + j] : j;
      if (e < 0 || e >= n_avail[s_id] || (mode == 0 && e >= t / ratio)) {
#pragma omp atomic write
        ok = 0;
        e = 0;
      }
      orc_load_entry(kv_fmt, D, R, P, kv_pool, pt, e, X + j * (int64_t)D);
    }
    for (int64_t j = 0; j < nw; ++j) {
      int64_t p = w0 + j;
      int64_t slot = ((int64_t)s_id * W + p % W) * D;
      double* x = X + (ne + j) * (int64_t)D;
      if (win_fmt == 0) for (int d = 0; d < D; ++d) x[d] = ((const float*)win)[slot + d];
      else for (int d = 0; d < D; ++d) x[d] = orc_bf16_decode(((const uint16_t*)win)[slot + d]);
    }
    if (!ok) bad = 1;
#pragma omp parallel
    {
      double* z = (double*)malloc(sizeof(double) * (nx > 0 ? nx : 1));
      double* qh = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
      for (int h = 0; h < nh; ++h) {
        orc_rmsnorm(D, q + (r * nh + h) * (int64_t)D, gq, eps, qh);
        if (R > 0) orc_rope(D, R, base, (double)t, 1, qh);
        double mx = sink[h];
        for (int64_t j = 0; j < nx; ++j) {
          double acc = 0;
          for (int d = 0; d < D; ++d) acc += qh[d] * X[j * (int64_t)D + d];
          z[j] = acc * scale;
          if (z[j] > mx) mx = z[j];
        }
        double den = exp(sink[h] - mx);
        double* o = out + (r * nh + h) * (int64_t)D;
        for (int d = 0; d < D; ++d) o[d] = 0;
        for (int64_t j = 0; j < nx; ++j) {
          double p = exp(z[j] - mx);
          den += p;
          for (int d = 0; d < D; ++d) o[d] += p * X[j * (int64_t)D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= den;
        if (R > 0) orc_rope(D, R, base, (double)t, -1, o);
        if (lse) lse[r * nh + h] = mx + log(den);
      }
      free(z);
      free(qh);
    }
  }
  free(X);
  return bad ? -1 : 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the later parallel regions (n >= 1); used to time the oracle on one core. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
