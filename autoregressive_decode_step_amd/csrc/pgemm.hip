// Prefill projections on gfx950 matrix cores: Y[m][n] = sum_k X[m][k] W[n][k] for a chunk of prompt rows.
//
// A prompt chunk is a batch of rows ("Inside the engine", "1. CausalLM: the forward path": the projections take
// the batched routes), large enough that every weight tile can be reused by many rows. So unlike the decode
// batch (skinny, one pass over the weights), the chunk is tiled in both directions: a workgroup (4 waves)
// owns a 128 x 128 tile of Y, stages 32-wide k slices of its 128 X rows and 128 W rows in LDS (two buffers:
// the next slice is loaded into registers while the current one is multiplied), and each wave multiplies a
// 64 x 64 sub-tile with v_mfma_f32_16x16x32_bf16 (4 x 4 tiles of 16 x 16). X is fp32 carried as bf16 hi + lo
// (each product taken twice into fp32), W is bf16 and exact. Where the tiles alone do not fill the chip, K is
// split: each split writes its partial tile, and the epilogue kernel adds the splits in order and applies the
// operation (store, residual add, SiLU-gate into hi/lo). Up to 64 rows (the decode batch) take 64 x 128 tiles.
//
// MFMA operands (per wave, 16 x 32 by 32 x 16): lane l holds row l % 16 of the X tile and row l % 16 of the
// W tile, eight consecutive k of group l / 16 (one 16-byte LDS read each); the 16 x 16 result gives lane l
// X rows 4 (l / 16) .. + 3 at W row l % 16.
#include <algorithm>

#include "kernels.h"

namespace llmk {

typedef __bf16 pg_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float pg_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int PG_THREADS = 256;
constexpr int PG_BM = 128;
constexpr int PG_BN = 128;
constexpr int PG_BK = 32;     // k per slice of 128-row tiles
constexpr int PG_BK64 = 64;   // k per slice of 64-row tiles

__device__ __forceinline__ pg_f32x4_t pg_mfma(const uint4& a, const uint4& b, const pg_f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pg_bf16x8_t, a),
                                                 __builtin_bit_cast(pg_bf16x8_t, b), c, 0, 0, 0);
}

// v where the mask is all ones, zero where it is zero (a per-word mask: a select of whole vectors would go
// through memory)
__device__ __forceinline__ uint4 pg_mask(const uint4& v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// W row n (clamped into [0, N)): rows [0, n0) of w0, then n1 rows of w1, then w2
__device__ __forceinline__ const bf16_t* pg_wrow(const PgemmParams& p, int64_t n) {
  const int64_t r = min(n, p.N - 1);
  if (r < p.n0) return static_cast<const bf16_t*>(p.w0) + r * p.K;
  if (r < p.n0 + p.n1) return static_cast<const bf16_t*>(p.w1) + (r - p.n0) * p.K;
  return static_cast<const bf16_t*>(p.w2) + (r - p.n0 - p.n1) * p.K;
}

// BM = 128: each wave multiplies a 64 x 64 sub-tile, slices of BK = 32. BM = 64 (a decode batch of up to 64
// rows): a 64 x 128 tile, each wave 64 x 32, so no matrix-core work goes to rows that do not exist, with slices
// of BK = 64 so twice the weight bytes are on their way per barrier.
template <int BM, int BK>
__global__ __launch_bounds__(PG_THREADS, BM == 64 ? 2 : 1) void pgemm_kernel(const PgemmParams p) {
  static_assert((BM == 64 || BM == 128) && BK % 32 == 0, "64 or 128 rows, k slices of 32 or more");
  constexpr int LDK = BK + 8;                        // LDS row stride in bf16 (80 or 144 bytes): the 16 rows
                                                     // one operand read touches use different banks
  constexpr int GPR = BK / 8;                        // 8-element groups per tile row
  constexpr int XG = BM * GPR / PG_THREADS;          // groups of the X tile per thread
  constexpr int WG = PG_BN * GPR / PG_THREADS;       // groups of the W tile per thread
  constexpr int WN = BM == 64 ? 4 : 2;               // waves along N
  constexpr int TN = PG_BN / WN / 16;                // 16-column tiles per wave
  __shared__ __align__(16) bf16_t s_a[2][2][BM][LDK];        // [buffer][hi, lo][row][k]
  __shared__ __align__(16) bf16_t s_w[2][PG_BN][LDK];        // [buffer][row][k]

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;                   // this wave's 64 x (16 TN) sub-tile
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * PG_BN;
  const int64_t kb = (int64_t)blockIdx.z * p.kslice;
  const int64_t ke = min(p.K, kb + p.kslice);
  const int nk = (int)((ke - kb + BK - 1) / BK);

  // staging: thread t moves 8-element groups g = t, t + 256, ... of each tile (row g / GPR, group g % GPR).
  // Two register sets in turn keep the loads of slice i + 2 in flight while slice i is multiplied and slice
  // i + 1 goes to LDS; every load is issued unconditionally (past the end of K, from k = 0) and zeroed when it
  // is staged, so no load sits in a branch of its own.
  const bf16_t* ah[XG];
  const bf16_t* al[XG];
  int xrow[XG], xk[XG];
#pragma unroll
  for (int i = 0; i < XG; ++i) {
    const int g = t + i * PG_THREADS;
    xrow[i] = g / GPR;
    xk[i] = (g % GPR) * 8;
    const int64_t m = min(m0 + xrow[i], (int64_t)p.M - 1);   // rows past M read a valid row; never stored
    ah[i] = p.ahi + m * p.lda;
    al[i] = p.alo + m * p.lda;
  }
  const bf16_t* wr[WG];
  int wrow[WG], wk[WG];
#pragma unroll
  for (int i = 0; i < WG; ++i) {
    const int g = t + i * PG_THREADS;
    wrow[i] = g / GPR;
    wk[i] = (g % GPR) * 8;
    wr[i] = pg_wrow(p, n0 + wrow[i]);
  }
  // a set's k: its groups past the end of K are zeroed when staged (K is a multiple of 8: a group is all in or
  // all out)
  uint4 xh[2][XG], xl[2][XG], wv[2][WG];
  int64_t ks[2] = {0, 0};
#define PG_LOAD(S, K)                                                                   \
  {                                                                                     \
    ks[S] = (K);                                                                        \
    _Pragma("unroll") for (int i = 0; i < XG; ++i) {                                    \
      const int64_t c = ks[S] + xk[i] < ke ? ks[S] + xk[i] : 0;                         \
      xh[S][i] = *reinterpret_cast<const uint4*>(ah[i] + c);                            \
      xl[S][i] = *reinterpret_cast<const uint4*>(al[i] + c);                            \
    }                                                                                   \
    _Pragma("unroll") for (int i = 0; i < WG; ++i) {                                    \
      const int64_t c = ks[S] + wk[i] < ke ? ks[S] + wk[i] : 0;                         \
      wv[S][i] = *reinterpret_cast<const uint4*>(wr[i] + c);                            \
    }                                                                                   \
  }
#define PG_STAGE(S, BUF)                                                                \
  {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < XG; ++i) {                                    \
      const uint32_t in = ks[S] + xk[i] < ke ? ~0u : 0u;                                \
      *reinterpret_cast<uint4*>(&s_a[BUF][0][xrow[i]][xk[i]]) = pg_mask(xh[S][i], in);   \
      *reinterpret_cast<uint4*>(&s_a[BUF][1][xrow[i]][xk[i]]) = pg_mask(xl[S][i], in);   \
    }                                                                                   \
    _Pragma("unroll") for (int i = 0; i < WG; ++i) {                                    \
      const uint32_t in = ks[S] + wk[i] < ke ? ~0u : 0u;                                \
      *reinterpret_cast<uint4*>(&s_w[BUF][wrow[i]][wk[i]]) = pg_mask(wv[S][i], in);      \
    }                                                                                   \
  }

  pg_f32x4_t acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = pg_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int orow = lane & 15, ok8 = (lane >> 4) * 8;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      uint4 wop[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        wop[j] = *reinterpret_cast<const uint4*>(&s_w[buf][wn * (16 * TN) + j * 16 + orow][kk + ok8]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 ah_ = *reinterpret_cast<const uint4*>(&s_a[buf][0][wm * 64 + i * 16 + orow][kk + ok8]);
        const uint4 al_ = *reinterpret_cast<const uint4*>(&s_a[buf][1][wm * 64 + i * 16 + orow][kk + ok8]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = pg_mfma(ah_, wop[j], acc[i][j]);
          acc[i][j] = pg_mfma(al_, wop[j], acc[i][j]);
        }
      }
    }
  };
  // slice i lives in LDS buffer i % 2 and comes through register set i % 2; at step i the set of slice i is
  // free again (its slice is in LDS) and takes slice i + 2, and the other set's slice i + 1 goes to the other
  // buffer, which was last read before the previous barrier
  // loads are issued every step (a slice past the last one reads the first again and is never staged), so
  // each set's registers live only from its load to its staging
  auto kof = [&](int i) { return i < nk ? kb + (int64_t)i * BK : kb; };
  PG_LOAD(0, kb)
  PG_LOAD(1, kof(1))
  if (nk > 0) PG_STAGE(0, 0)
  __syncthreads();
  for (int it = 0; it < nk; it += 2) {
    PG_LOAD(0, kof(it + 2))
    multiply(0);
    if (it + 1 < nk) PG_STAGE(1, 1)
    __syncthreads();
    if (it + 1 < nk) {
      PG_LOAD(1, kof(it + 3))
      multiply(1);
      if (it + 2 < nk) PG_STAGE(0, 0)
      __syncthreads();
    }
  }
#undef PG_LOAD
#undef PG_STAGE

  // this split's partial tile: lane l holds rows 4 (l / 16) .. + 3 of each 16-row tile at column l % 16
  float* y = p.y + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * (16 * TN) + j * 16 + orow;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        if (m < p.M && n < p.N) y[m * p.N + n] = acc[i][j][e];
      }
    }
}

// ---- decode batches (up to 64 rows): every weight byte once, straight into matrix-core operand registers ----
//
// With 64 rows a weight tile is used by one row block only, so nothing is gained by staging it in LDS, and a
// tile kernel that does so keeps one 64-wide k slice of weights in flight per workgroup between its barriers
// (about 32 KB a CU, far short of what HBM latency needs). Here each wave streams its own TN tiles of 16
// weight rows for the split's whole k range as B operands of v_mfma_f32_16x16x32_bf16 (lane l: row l % 16,
// k group l / 16, one 16-byte load), through a ring of 2 SG_KS TN loads that is refilled as it is read, the
// same way the batch-1 step streams its rows: 8 waves keep 16 KB each in flight. Only the activations (64 rows
// of bf16 hi + lo) go through LDS, in chunks of SG_KC k shared by the waves, one barrier a chunk; they are
// re-read from L2 once per 128 TN columns. Each product is taken for hi and lo into fp32 like the tile kernel.
constexpr int SG_THREADS = 512;
constexpr int SG_WAVES = SG_THREADS / 64;
constexpr int SG_KC = 128;                 // k per chunk of activations in LDS
constexpr int SG_KS = SG_KC / 32;          // matrix-core k steps per chunk
constexpr int SG_LDX = SG_KC + 8;          // LDS row stride of a chunk in bf16 (272 bytes)
constexpr int SG_XV = 2 * 64 * SG_KC / 8 / SG_THREADS;   // 16-byte groups of a chunk (hi and lo) per thread
constexpr int SG_CPT = SG_WAVES * 16;      // columns per workgroup and column tile of a wave

template <int TN>
__global__ __launch_bounds__(SG_THREADS, 1) void sgemm_kernel(const PgemmParams p) {
  constexpr int PER = SG_KS * TN;          // ring slots a chunk takes (k step major, then column tile)
  constexpr int RC = TN >= 4 ? 1 : 2;      // chunks of weight loads the ring holds ahead
  constexpr int R = RC * PER;
  __shared__ __align__(16) bf16_t s_x[2][2][64][SG_LDX];   // [buffer][hi, lo][row][k]

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t kb = (int64_t)blockIdx.z * p.kslice;
  const int64_t ke = min(p.K, kb + p.kslice);
  const int nc = (int)((ke - kb + SG_KC - 1) / SG_KC);
  const int64_t nb = ((int64_t)blockIdx.x * SG_WAVES + wave) * 16 * TN;   // this wave's first column
  // the workgroups of a split do not all start at the same k: chunk c is chunk (c + rot) % nc of the split
  const int rot = (int)(blockIdx.x % (unsigned)nc);
  auto chunk_k = [&](int c) { return kb + (int64_t)((c + rot) % nc) * SG_KC; };

  // this lane's weight row of each column tile (rows past N read row N - 1 and are never stored) and k group
  const bf16_t* wrow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) wrow[j] = pg_wrow(p, nb + 16 * j + (lane & 15));
  const int kg = 8 * (lane >> 4);
  // weight load of k step s (counted from kb) of column tile j; past ke it reads k = 0 (its products meet
  // activations that are zero there)
  auto wload = [&](int s, int j) {
    const int64_t k = chunk_k(s / SG_KS) + 32 * (int64_t)(s % SG_KS) + kg;
    return *reinterpret_cast<const uint4*>(wrow[j] + (k < ke ? k : 0));
  };

  // activation chunk c: thread t moves groups g = t + 512 i (hi for g < 1024, then lo): row (g % 1024) / 16,
  // k group g % 16; rows past M read row M - 1, groups past ke are zeroed when stored
  uint4 xr[SG_XV];
  auto xload = [&](int c) {
    const int64_t k0 = chunk_k(c < nc ? c : 0);
#pragma unroll
    for (int i = 0; i < SG_XV; ++i) {
      const int g = t + i * SG_THREADS, rem = g & 1023;
      const int64_t m = min(rem >> 4, p.M - 1);
      const int64_t k = k0 + 8 * (rem & 15);
      xr[i] = *reinterpret_cast<const uint4*>((g < 1024 ? p.ahi : p.alo) + m * p.lda + (k < ke ? k : 0));
    }
  };
  auto xstore = [&](int c, int buf) {
    const int64_t k0 = c < nc ? chunk_k(c) : ke;   // past the last chunk: all zero
#pragma unroll
    for (int i = 0; i < SG_XV; ++i) {
      const int g = t + i * SG_THREADS, rem = g & 1023;
      const uint32_t in = k0 + 8 * (rem & 15) < ke ? ~0u : 0u;
      *reinterpret_cast<uint4*>(&s_x[buf][g >> 10][rem >> 4][8 * (rem & 15)]) = pg_mask(xr[i], in);
    }
  };

  pg_f32x4_t acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = pg_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // prologue: chunk 0's activations, then the first two chunks' weight loads
  uint4 ring[R];
  xload(0);
  xstore(0, 0);
#pragma unroll
  for (int q = 0; q < R; ++q) ring[q] = wload(q / TN, q % TN);   // chunks 0 .. RC - 1
  __syncthreads();

  // chunk c in buffer B, its weights in ring half H: the next chunk's activations are loaded first (so that
  // waiting for them later waits for none of the weight loads issued after), every slot is refilled with the
  // same slot two chunks on as soon as it is read, and loads past the last chunk re-read valid addresses
  auto chunk = [&](int c, int B, int H) __attribute__((always_inline)) {
    xload(c + 1);
#pragma unroll
    for (int s = 0; s < SG_KS; ++s) {
      uint4 ah[4], al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ah[i] = *reinterpret_cast<const uint4*>(&s_x[B][0][16 * i + (lane & 15)][32 * s + kg]);
        al[i] = *reinterpret_cast<const uint4*>(&s_x[B][1][16 * i + (lane & 15)][32 * s + kg]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int q = (H % RC) * PER + s * TN + j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i][j] = pg_mfma(ah[i], ring[q], acc[i][j]);
          acc[i][j] = pg_mfma(al[i], ring[q], acc[i][j]);
        }
        // the refill reuses the slot's registers once its products are issued, and goes out here rather than
        // after the chunk's products (where the scheduler would move it, and the ring would run dry each chunk)
        ring[q] = wload((c + RC < nc ? c + RC : 0) * SG_KS + s, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    xstore(c + 1, B ^ 1);
    __syncthreads();
  };
  // chunks in pairs with nothing conditional in the loop, so that every slot's wait counts exactly the loads
  // issued after it (an odd last chunk is followed by one whose activations are all zero)
  for (int c = 0; c < nc; c += 2) {
    chunk(c, 0, 0);
    chunk(c + 1, 1, 1);
  }

  // this split's partial tile: lane l holds rows 4 (l / 16) .. + 3 of each 16-row tile at column l % 16
  float* y = p.y + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = nb + 16 * j + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = 16 * i + (lane >> 4) * 4 + e;
        if (m < p.M && n < p.N) y[m * p.N + n] = acc[i][j][e];
      }
    }
}

// the splits' sum of element (m, n), in split order
__device__ __forceinline__ float pg_sum(const PgemmParams& p, int64_t m, int64_t n) {
  float v = 0.0f;
  for (int z = 0; z < p.ksplit; ++z) v += p.y[((int64_t)z * p.M + m) * p.N + n];
  return v;
}

__global__ void pgemm_epilogue_kernel(const PgemmParams p, int mode) {
  const int64_t cols = mode == PG_GATEUP ? p.N / 2 : p.N;
  const int64_t total = (int64_t)p.M * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / cols, n = i % cols;
    if (mode == PG_STORE) {
      p.out[m * p.ldo + n] = pg_sum(p, m, n);
    } else if (mode == PG_RESID) {
      const float xo = p.out[m * p.ldo + n] + pg_sum(p, m, n);
      p.out[m * p.ldo + n] = xo;
      if (p.hidden) p.hidden[m * p.hidden_stride + n] = xo;
    } else {   // PG_GATEUP: gate rows first, then the same number of up rows
      const float u = silu_f(pg_sum(p, m, n)) * pg_sum(p, m, n + cols);
      bf16_t hi, lo;
      split_bf16(u, hi, lo);
      p.uhi[m * cols + n] = hi;
      p.ulo[m * cols + n] = lo;
    }
  }
}

// The same, four columns per thread: grid (column blocks of 1,024, rows); needs the column count, the row
// strides and every buffer to allow 16-byte accesses (8-byte for the hi/lo outputs).
__global__ __launch_bounds__(256) void pgemm_epilogue4_kernel(const PgemmParams p, int mode) {
  const int64_t cols = mode == PG_GATEUP ? p.N / 2 : p.N;
  const int64_t m = blockIdx.y;
  const int64_t n = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (n >= cols) return;
  auto sum4 = [&](int64_t c) {
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int z = 0; z < p.ksplit; ++z) {
      const float4 y = *reinterpret_cast<const float4*>(p.y + ((int64_t)z * p.M + m) * p.N + c);
      v.x += y.x;
      v.y += y.y;
      v.z += y.z;
      v.w += y.w;
    }
    return v;
  };
  if (mode == PG_STORE) {
    *reinterpret_cast<float4*>(p.out + m * p.ldo + n) = sum4(n);
  } else if (mode == PG_RESID) {
    const float4 y = sum4(n);
    float4 x = *reinterpret_cast<const float4*>(p.out + m * p.ldo + n);
    x.x += y.x;
    x.y += y.y;
    x.z += y.z;
    x.w += y.w;
    *reinterpret_cast<float4*>(p.out + m * p.ldo + n) = x;
    if (p.hidden) *reinterpret_cast<float4*>(p.hidden + m * p.hidden_stride + n) = x;
  } else {   // PG_GATEUP
    const float4 g = sum4(n), u = sum4(n + cols);
    const float e[4] = {silu_f(g.x) * u.x, silu_f(g.y) * u.y, silu_f(g.z) * u.z, silu_f(g.w) * u.w};
    bf16_t h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) split_bf16(e[k], h[k], l[k]);
    *reinterpret_cast<uint2*>(p.uhi + m * cols + n) =
        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    *reinterpret_cast<uint2*>(p.ulo + m * cols + n) =
        make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
  }
}

// rows per tile: 64 for up to 64 rows (a decode batch, a short last prompt chunk), else 128; k per slice
static int pg_bm(int32_t M) { return M <= 64 ? 64 : PG_BM; }
static int pg_bk(int32_t M) { return M <= 64 ? PG_BK64 : PG_BK; }

// Rows up to 64 with at least 64 groups of 256 columns (gate|up, the head) take the register-streamed kernel;
// narrower ones (q|k|v, o, down), which it could only fill with many short k splits, the 64 x 128 tiles.
static bool sg_use(int32_t M, int64_t N) { return M <= 64 && N >= 64 * 2 * SG_CPT; }
// column tiles per wave: 2, or 4 where 2 would give more column groups than the 256 CUs hold at once (the
// vocabulary head: one round of workgroups instead of two; measured 255 against 272 us on the 8B head)
static int sg_tn(int64_t N) { return (N + 2 * SG_CPT - 1) / (2 * SG_CPT) > 256 ? 4 : 2; }

void pgemm_plan(PgemmParams& p, int target_blocks) {
  if (sg_use(p.M, p.N)) {
    // column groups of 256, k split in whole chunks (at least two a split) so that the workgroups, one a CU,
    // fit the target at once
    const int tn = sg_tn(p.N);
    const int64_t groups = (p.N + tn * SG_CPT - 1) / (tn * SG_CPT);
    const int64_t chunks = (p.K + SG_KC - 1) / SG_KC;
    int64_t ks = (int64_t)target_blocks / groups;
    ks = std::max<int64_t>(1, std::min<int64_t>(ks, chunks / 2));
    p.kslice = (chunks + ks - 1) / ks * SG_KC;
    p.ksplit = (int32_t)((p.K + p.kslice - 1) / p.kslice);
    return;
  }
  const int64_t tiles = ((p.N + PG_BN - 1) / PG_BN) * ((p.M + pg_bm(p.M) - 1) / pg_bm(p.M));
  int64_t ks = (target_blocks + tiles - 1) / tiles;
  const int bk = pg_bk(p.M);
  const int64_t steps = (p.K + bk - 1) / bk;
  ks = std::max<int64_t>(1, std::min<int64_t>(ks, steps / 8));   // at least 8 k slices per split
  int64_t slice = (steps + ks - 1) / ks * bk;
  p.kslice = slice;
  p.ksplit = (int32_t)((p.K + slice - 1) / slice);
}

hipError_t pgemm_launch(const PgemmParams& p, int mode, hipStream_t s) {
  if (p.M < 1 || p.K % 8 != 0) return hipErrorInvalidValue;
  if (sg_use(p.M, p.N)) {
    if (p.kslice % SG_KC != 0) return hipErrorInvalidValue;
    const int tn = sg_tn(p.N);
    const dim3 grid((unsigned)((p.N + tn * SG_CPT - 1) / (tn * SG_CPT)), 1, (unsigned)p.ksplit);
    if (tn == 4)
      hipLaunchKernelGGL(sgemm_kernel<4>, grid, dim3(SG_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL(sgemm_kernel<2>, grid, dim3(SG_THREADS), 0, s, p);
  } else {
    if (p.kslice % pg_bk(p.M) != 0) return hipErrorInvalidValue;
    const int bm = pg_bm(p.M);
    const dim3 grid((unsigned)((p.N + PG_BN - 1) / PG_BN), (unsigned)((p.M + bm - 1) / bm), (unsigned)p.ksplit);
    if (bm == 64)
      hipLaunchKernelGGL((pgemm_kernel<64, PG_BK64>), grid, dim3(PG_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL((pgemm_kernel<128, PG_BK>), grid, dim3(PG_THREADS), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mode == PG_NONE) return e;
  const int64_t cols = mode == PG_GATEUP ? p.N / 2 : p.N;
  auto al = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; };
  const bool vec = cols % 4 == 0 && p.N % 4 == 0 && al(p.y, 16) && p.M <= 65535 &&
                   (mode == PG_GATEUP ? al(p.uhi, 8) && al(p.ulo, 8)
                                      : p.ldo % 4 == 0 && al(p.out, 16) &&
                                            (!p.hidden || (al(p.hidden, 16) && p.hidden_stride % 4 == 0)));
  if (vec) {
    const dim3 grid((unsigned)((cols + 1023) / 1024), (unsigned)p.M);
    hipLaunchKernelGGL(pgemm_epilogue4_kernel, grid, dim3(256), 0, s, p, mode);
    return hipGetLastError();
  }
  const int64_t total = (int64_t)p.M * cols;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(pgemm_epilogue_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, mode);
  return hipGetLastError();
}

}  // namespace llmk
