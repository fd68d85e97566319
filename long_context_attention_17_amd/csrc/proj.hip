// The attention sublayer around CSA / HCA: the low-rank query projections and the
// grouped output projection (dsv4 book Ch.6 "Low-rank query generation", "The
// lightning indexer" and "Grouped output projections"; Ch.4 "Query head scaling and
// grouped output projections").  All of it is dense bf16 contraction, run here on
// one hand-written MFMA GEMM, C[m, n] = sum_k A[m, k] W[n, k] (both operands
// K-contiguous, fp32 accumulation):
//   - up to two N segments per launch that share A (W^DQ and W^w both read h; W^UQ
//     and W^IUQ both read the latent), each with its own weights and output;
//   - a batch dimension with strides (the g group projections of the output);
//   - a K split into fp32 partials, added in split order by a second kernel, when the
//     output alone has too few tiles to fill the chip (decode-sized M).
#include "common.h"
#include "kernels.h"

namespace ca {

namespace {

constexpr int kGroupM = 8;                           // M tiles per group of the tile order

// Workgroup tile MT x NT of WAVES wavefronts, one K tile of register prefetch (M <= 32 runs
// gemm_skinny_kernel below instead):
//   128 x 128, 4 wavefronts (2 x 2 of 64 x 64): two workgroups per CU, one's barrier and LDS
//     stores overlapping the other's MFMAs;
//   256 x 256, 8 wavefronts (2 x 4 of 128 x 64): one workgroup per CU, two wavefronts per
//     SIMD; each A fragment read from LDS feeds two MFMAs and each W fragment four.
//   (256 x 128 with 4 wavefronts, one per SIMD, measured slower: 420 vs 727 TF/s.)
template <int MT, int NT, int KT, int WAVES = 4>
struct GemmShape {
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kP = KT + 8;                                   // LDS row pitch (bf16)
  static constexpr int kWavesM = MT >= 128 ? 2 : 1, kWavesN = WAVES / kWavesM;
  static constexpr int kWM = MT / kWavesM, kWN = NT / kWavesN;       // one wavefront's tile
  static constexpr int kBM = kWM / 32, kBN = kWN / 32;                // 32x32 MFMA blocks per wavefront
  static constexpr int kAChunks = MT * KT / 8 / kThreads;             // 16-byte loads per thread
  static constexpr int kWChunks = NT * KT / 8 / kThreads;
  static constexpr int kPF = 1;
  static constexpr int kCPitch = NT + 8;                              // bf16 output staging row pitch
};

// Rows row0 .. of a K-contiguous operand, columns k0 .. k0 + KT - 1, into registers:
// chunk i = threadIdx.x + 256 j is row i / (KT / 8), columns 8 (i % (KT / 8)) .. +7.  Rows
// past max_row re-read the last row (their products land in rows / columns never stored).
template <int NCH, int KT, int NT_ = 256>
__device__ __forceinline__ void tile_load(const uint16_t* base, int64_t ld, int row0, int max_row, int k0,
                                          u32x4* regs) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int i = threadIdx.x + NT_ * j;
    int r = row0 + i / (KT / 8);
    r = r < max_row ? r : max_row - 1;
    regs[j] = *(const u32x4*)(base + (int64_t)r * ld + k0 + 8 * (i % (KT / 8)));
  }
}

template <int NCH, int KT, int NT_ = 256>
__device__ __forceinline__ void tile_store(uint16_t* lds, const u32x4* regs) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int i = threadIdx.x + NT_ * j;
    *(u32x4*)(lds + (i / (KT / 8)) * (KT + 8) + 8 * (i % (KT / 8))) = regs[j];
  }
}

struct TileCoord {
  int b, s, m_tile, n_tile;
};

// Block -> tile.  Blocks are dealt to the 8 XCDs round robin; block id i runs on XCD i % 8,
// so the logical tile is taken as (i % 8) * per_xcd + i / 8: each XCD walks its own
// contiguous range of the tile order, and within it groups of kGroupM M tiles sweep the N
// tiles together (an N tile of W is reused by kGroupM neighbours in the XCD's L2).
__device__ __forceinline__ bool tile_of(const GemmArgs& g, TileCoord& t) {
  const int64_t id = blockIdx.x;
  const int64_t per_xcd = g.grid_blocks / 8;
  const int64_t u_all = (id % 8) * per_xcd + id / 8;
  const int64_t per_z = (int64_t)g.m_tiles * g.n_tiles;
  if (u_all >= per_z * g.batch * g.k_splits) return false;
  const int z = (int)(u_all / per_z);
  const int64_t u = u_all % per_z;
  const int64_t in_group = (int64_t)kGroupM * g.n_tiles;
  const int first_m = (int)(u / in_group) * kGroupM;
  const int gsize = min(g.m_tiles - first_m, kGroupM);
  t.m_tile = first_m + (int)((u % in_group) % gsize);
  t.n_tile = (int)((u % in_group) / gsize);
  t.b = z / g.k_splits;
  t.s = z % g.k_splits;
  return true;
}

template <int MT, int NT, int KT, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) gemm_nt_kernel(GemmArgs g) {
  using S = GemmShape<MT, NT, KT, WAVES>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (MT + NT) * S::kP];
  uint16_t* As[2] = {smem, smem + MT * S::kP};                    // A tiles, then W tiles
  uint16_t* Ws[2] = {smem + 2 * MT * S::kP, smem + (2 * MT + NT) * S::kP};
  TileCoord tc;
  if (!tile_of(g, tc)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;
  const int sg = tc.n_tile >= g.seg[0].n_tiles ? 1 : 0;
  const GemmSeg& seg = g.seg[sg];
  const int m0 = tc.m_tile * MT, n0 = (tc.n_tile - (sg ? g.seg[0].n_tiles : 0)) * NT;
  const uint16_t* A = (const uint16_t*)g.A + tc.b * g.a_batch;
  const uint16_t* W = (const uint16_t*)seg.W + tc.b * seg.w_batch;
  const int kt0 = (int)((int64_t)tc.s * g.k_tiles / g.k_splits);
  const int n_kt = (int)((int64_t)(tc.s + 1) * g.k_tiles / g.k_splits) - kt0;

  f32x16 acc[S::kBM][S::kBN];
#pragma unroll
  for (int i = 0; i < S::kBM; ++i)
#pragma unroll
    for (int j = 0; j < S::kBN; ++j) acc[i][j] = f32x16{};

  // register stages of the K tiles in flight (PF of them)
  u32x4 ra[S::kPF][S::kAChunks], rw[S::kPF][S::kWChunks];
  auto load = [&](int p, int i) {
    tile_load<S::kAChunks, KT, S::kThreads>(A, g.lda, m0, g.M, (kt0 + i) * KT, ra[p]);
    tile_load<S::kWChunks, KT, S::kThreads>(W, seg.ldw, n0, seg.N, (kt0 + i) * KT, rw[p]);
  };
  auto store = [&](int p, int buf) {
    tile_store<S::kAChunks, KT, S::kThreads>(As[buf], ra[p]);
    tile_store<S::kWChunks, KT, S::kThreads>(Ws[buf], rw[p]);
  };
  auto mfmas = [&](int buf) {
    const uint16_t* as = As[buf] + (wm * S::kWM + (lane & 31)) * S::kP + 8 * (lane >> 5);
    const uint16_t* ws = Ws[buf] + (wn * S::kWN + (lane & 31)) * S::kP + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < KT; kk += 16) {
      bf16x8 af[S::kBM], wf[S::kBN];
#pragma unroll
      for (int i = 0; i < S::kBM; ++i) af[i] = *(const bf16x8*)(as + 32 * i * S::kP + kk);
#pragma unroll
      for (int j = 0; j < S::kBN; ++j) wf[j] = *(const bf16x8*)(ws + 32 * j * S::kP + kk);
#pragma unroll
      for (int i = 0; i < S::kBM; ++i)
#pragma unroll
        for (int j = 0; j < S::kBN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
  };

  // K tile i sits in register stage i % PF until it is stored to LDS buffer i % 2
  load(0, 0);
  if (S::kPF > 1 && n_kt > 1) load(S::kPF - 1, 1);
  store(0, 0);
  __syncthreads();
  // step i (c = i % 2, a constant in each unrolled copy): refill the register stage that
  // tile i left for tile i + PF, multiply tile i, store tile i + 1, barrier
  auto step = [&](int i, int c) {
    if (i + S::kPF < n_kt) load(S::kPF > 1 ? c : 0, i + S::kPF);
    mfmas(c);
    if (i + 1 < n_kt) store(S::kPF > 1 ? c ^ 1 : 0, c ^ 1);
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < n_kt; i += 2) {
    step(i, 0);
    step(i + 1, 1);
  }
  if (i < n_kt) step(i, 0);

  // acc[i][j] element v of lane l: row 32 i + 8 (v / 4) + 4 (l / 32) + v % 4 and column
  // 32 j + l % 32 of the wavefront's tile
  const int mw = wm * S::kWM + 4 * (lane >> 5), nw = wn * S::kWN + (lane & 31);
  if (g.k_splits == 1 && !seg.c_f32) {
    // bf16 output: the tile goes through LDS (free after the last barrier) so that the global
    // stores are 16-byte runs along the rows of C
    static_assert(MT * S::kCPitch <= 2 * (MT + NT) * S::kP, "output staging fits the operand buffers");
    uint16_t* ct = smem;
#pragma unroll
    for (int i2 = 0; i2 < S::kBM; ++i2)
#pragma unroll
      for (int j = 0; j < S::kBN; ++j) {
        const f32x16 blk = acc[i2][j];
#pragma unroll
        for (int v = 0; v < 16; ++v)
          ct[(mw + 32 * i2 + 8 * (v >> 2) + (v & 3)) * S::kCPitch + nw + 32 * j] = f32_to_bf16_bits(blk[v]);
      }
    __syncthreads();
    uint16_t* cbase = (uint16_t*)seg.C + tc.b * seg.c_batch;
    const bool vec = ((seg.ldc | tc.b * seg.c_batch) & 7) == 0 && ((uintptr_t)seg.C & 15) == 0;
    constexpr int kChunksRow = NT / 8;
#pragma unroll
    for (int p = 0; p < MT * kChunksRow / S::kThreads; ++p) {
      const int q = threadIdx.x + S::kThreads * p, r = q / kChunksRow, c = 8 * (q % kChunksRow);
      const int m = m0 + r, n = n0 + c;
      if (m >= g.M || n >= seg.N) continue;
      const u32x4 x = *(const u32x4*)(ct + r * S::kCPitch + c);
      uint16_t* dst = cbase + (int64_t)m * seg.ldc + n;
      if (vec && n + 8 <= seg.N) {
        *(u32x4*)dst = x;
      } else {
        for (int e = 0; e < 8 && n + e < seg.N; ++e) dst[e] = (uint16_t)(x[e >> 1] >> (16 * (e & 1)));
      }
    }
    return;
  }
  const int64_t part_base = seg.part_off + ((int64_t)tc.s * g.batch + tc.b) * g.M * seg.N;
#pragma unroll
  for (int i2 = 0; i2 < S::kBM; ++i2)
#pragma unroll
    for (int j = 0; j < S::kBN; ++j) {
      const f32x16 blk = acc[i2][j];
      const int n = n0 + nw + 32 * j;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + mw + 32 * i2 + 8 * (v >> 2) + (v & 3);
        if (m < g.M && n < seg.N) {
          if (g.k_splits > 1) g.part[part_base + (int64_t)m * seg.N + n] = blk[v];
          else ((float*)seg.C)[tc.b * seg.c_batch + (int64_t)m * seg.ldc + n] = blk[v];
        }
      }
    }
}

// Decode-sized M (<= 32 MB): no LDS and no barriers.  Wavefront w of the workgroup owns output
// columns n0 + 32 w .. +31 (MB 32 x 32 MFMA blocks, one per 32 rows; each W fragment feeds
// all of them) and reads its operands straight from
// global memory in the MFMA lane layout, a K group of 64 at a time: lane l holds row / column
// l % 32 and the 32 contiguous elements 32 (l / 32) .. +31 of the group (64 bytes), which
// feed four MFMAs (step s takes elements 8 s .. 8 s + 7 of each half: the same permutation of
// K on both operands).  PF groups stay in flight per wavefront, so the weights stream with
// many bytes outstanding per CU.
template <int PF, int MB>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(GemmArgs g) {
  TileCoord tc;
  if (!tile_of(g, tc)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sg = tc.n_tile >= g.seg[0].n_tiles ? 1 : 0;
  const GemmSeg& seg = g.seg[sg];
  const int n0 = (tc.n_tile - (sg ? g.seg[0].n_tiles : 0)) * 128 + 32 * wave;
  if (n0 >= seg.N) return;                               // (wavefront-uniform; no barriers follow)
  const int kg0 = (int)((int64_t)tc.s * g.k_tiles / g.k_splits);   // K groups of 64
  const int n_kg = (int)((int64_t)(tc.s + 1) * g.k_tiles / g.k_splits) - kg0;
  const int nr = min(n0 + (lane & 31), seg.N - 1);
  const uint16_t* wrow = (const uint16_t*)seg.W + tc.b * seg.w_batch + (int64_t)nr * seg.ldw + 32 * (lane >> 5) +
                         (int64_t)kg0 * 64;
  const uint16_t* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    arow[mb] = (const uint16_t*)g.A + tc.b * g.a_batch + (int64_t)min(32 * mb + (lane & 31), g.M - 1) * g.lda +
               32 * (lane >> 5) + (int64_t)kg0 * 64;
  u32x4 wv[PF][4], av[PF][MB][4];
  auto load = [&](int p, int i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wv[p][q] = *(const u32x4*)(wrow + (int64_t)i * 64 + 8 * q);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[p][mb][q] = *(const u32x4*)(arow[mb] + (int64_t)i * 64 + 8 * q);
    }
  };
  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < n_kg) load(p, p);
  // group i sits in register stage i % PF (a constant in each unrolled copy)
  auto step = [&](int i, int c) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[c][mb][q]),
                                                          __builtin_bit_cast(bf16x8, wv[c][q]), acc[mb], 0, 0, 0);
    if (i + PF < n_kg) load(c, i + PF);
  };
  int i = 0;
  for (; i + PF <= n_kg; i += PF)
#pragma unroll
    for (int c = 0; c < PF; ++c) step(i + c, c);
#pragma unroll
  for (int c = 0; c < PF; ++c)
    if (i + c < n_kg) step(i + c, c);
  // acc[mb] element v of lane l: row 32 mb + 8 (v / 4) + 4 (l / 32) + v % 4, column n0 + l % 32
  const int n = n0 + (lane & 31);
  if (n >= seg.N) return;
  const int64_t part_base = seg.part_off + ((int64_t)tc.s * g.batch + tc.b) * g.M * seg.N;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const f32x16 blk = acc[mb];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 32 * mb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (m < g.M) {
        if (g.k_splits > 1) g.part[part_base + (int64_t)m * seg.N + n] = blk[v];
        else if (seg.c_f32) ((float*)seg.C)[tc.b * seg.c_batch + (int64_t)m * seg.ldc + n] = blk[v];
        else ((uint16_t*)seg.C)[tc.b * seg.c_batch + (int64_t)m * seg.ldc + n] = f32_to_bf16_bits(blk[v]);
      }
    }
  }
}

// C_b[m, n] = sum_s part[s][b][m][n], the splits added in order; both segments.
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmArgs g) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int sg = 0;
  const int64_t n0 = (int64_t)g.batch * g.M * g.seg[0].N;
  if (i >= n0) {
    i -= n0;
    sg = 1;
    if (g.n_seg < 2 || i >= (int64_t)g.batch * g.M * g.seg[1].N) return;
  }
  const GemmSeg& seg = g.seg[sg];
  const int64_t per = (int64_t)g.M * seg.N;
  const int64_t b = i / per, mn = i % per, m = mn / seg.N, n = mn % seg.N;
  const float* p = g.part + seg.part_off + b * per + mn;
  float v = 0.0f;
  for (int s = 0; s < g.k_splits; ++s) v += p[(int64_t)s * g.batch * per];
  const int64_t o = b * seg.c_batch + m * seg.ldc + n;
  if (seg.c_f32) ((float*)seg.C)[o] = v;
  else ((uint16_t*)seg.C)[o] = f32_to_bf16_bits(v);
}

// Workgroup tile: M <= 32 runs gemm_skinny_kernel (32 rows, 128 columns, K groups of 64); a
// 64-row skinny variant measured slower than the 128-row tile at 64 rows (1.97 vs 2.26 TB/s of
// weights).  Otherwise 256 x 256 (eight wavefronts, one workgroup per CU) when that still
// makes at least kBigTiles tiles, else 128 x 128: the big tile reads half the LDS bytes per
// MFMA (7-16 % faster at 32K tokens) but idles CUs when tiles are few (Flash output
// projection at 4K tokens: 0.77 -> 1.02 ms).
constexpr int kSkinnyPF = 2;
constexpr int64_t kBigTiles = 1024;
void tile_of_gemm(const GemmArgs& g, int* tm, int* tn) {
  if (g.M <= 32) {
    *tm = 32;
    *tn = 128;
    return;
  }
  int64_t n256 = 0;
  for (int q = 0; q < g.n_seg; ++q) n256 += (g.seg[q].N + 255) / 256;
  const bool big = (int64_t)((g.M + 255) / 256) * n256 * g.batch >= kBigTiles;
  *tm = *tn = big ? 256 : 128;
}

}  // namespace

void gemm_plan(GemmArgs& g) {
  int mt, nt;
  tile_of_gemm(g, &mt, &nt);
  g.tile_m = mt;
  g.tile_n = nt;
  constexpr int kt = 64;
  g.m_tiles = (g.M + mt - 1) / mt;
  g.n_tiles = 0;
  for (int s = 0; s < 2; ++s) {
    g.seg[s].n_tiles = s < g.n_seg ? (g.seg[s].N + nt - 1) / nt : 0;
    g.n_tiles += g.seg[s].n_tiles;
  }
  g.k_tiles = g.K / kt;
  const int64_t tiles = (int64_t)g.m_tiles * g.n_tiles * g.batch;
  // K splits until the launch has ~1,000 workgroups (four per CU; decode-sized M: ~512, as
  // each streams its weights with many loads in flight and fewer splits write fewer
  // partials), each split keeping at least 256 of K
  int s = 1;
  while (tiles * s < (mt == 32 ? 512 : 1024) && 2 * s * 256 <= g.k_tiles * kt && s < 32) s *= 2;
  g.k_splits = s;
  int64_t off = 0;
  for (int q = 0; q < g.n_seg; ++q) {
    g.seg[q].part_off = off;
    off += s > 1 ? (int64_t)s * g.batch * g.M * g.seg[q].N : 0;
  }
  g.part_floats = off;
  const int64_t total = tiles * s;
  g.grid_blocks = (total + 7) / 8 * 8;
}

hipError_t launch_gemm(GemmArgs g, hipStream_t st) {
  if (g.M == 0) return hipSuccess;
  gemm_plan(g);
  if (g.n_tiles == 0) return hipSuccess;
  if (g.k_splits > 1 && g.part == nullptr) return hipErrorInvalidValue;
  if (g.grid_blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipEvent_t ev0, ev1;
  timer_events(CA_TIMED_PROJ_GEMM, st, &ev0, &ev1);
  const dim3 grid((unsigned)g.grid_blocks);
  if (g.tile_m == 32) CA_LAUNCH((gemm_skinny_kernel<kSkinnyPF, 1>), grid, dim3(256), 0, st, ev0, ev1, g);
  else if (g.tile_m == 256) CA_LAUNCH((gemm_nt_kernel<256, 256, 64, 8>), grid, dim3(512), 0, st, ev0, ev1, g);
  else CA_LAUNCH((gemm_nt_kernel<128, 128, 64, 4>), grid, dim3(256), 0, st, ev0, ev1, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.k_splits == 1) return e;
  int64_t n = 0;
  for (int q = 0; q < g.n_seg; ++q) n += (int64_t)g.batch * g.M * g.seg[q].N;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace ca
