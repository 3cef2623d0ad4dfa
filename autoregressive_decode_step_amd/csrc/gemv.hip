// Bandwidth-bound GEMV kernels for gfx950.
//
// gemv_t_kernel: y = A^T x with A [K][N] row-major (the transposed form every per-layer projection of
// the decode step uses; llmk page, "A parallel path for one frozen kernel's known-slow shape").
//   - A workgroup (4 waves) owns a strip of 64*VEC output columns and a range of rows. Each lane owns
//     VEC adjacent columns and streams them down its wave's rows with 16-byte loads, so one wave reads
//     a contiguous 1 KiB segment of each row (fully coalesced), with two batches of rows in flight.
//   - The first batch of weight loads is issued before the input is read, so the prologue (loading the
//     input vector and, when fused, its RMSNorm) overlaps the first HBM round trip. Input values reach
//     the FMAs through readlane (a scalar operand), never through LDS.
//   - Waves reduce through LDS in a fixed order; workgroups that split K write fp32 partials and the
//     last workgroup of a column strip (an atomic ticket, release/acquire fences) sums them in split
//     order and runs the fused epilogue. No float atomics: results are bit-identical run to run.
//   - Epilogues: plain store; residual add (x = base + y, base may be the embedding row); SiLU-gate
//     (u = silu(gate) * up, gate and up streamed by the same lanes); q|k|v with RoPE on q and k and the
//     k, v append into the slot's K/V buffers (rounded to the pool dtype).
//
// head_kernel: y[r] = W[r] . h for W [rows][cols] (the untransposed output head), h = rmsnorm(x)*gain
// computed per wave while the first rows are in flight, one wave per group of rows, wave-shuffle
// reductions, and pass 1 of the greedy argmax fused into the same launch (pass 2 by the last
// workgroup; ties to the lower index, NaN first).
#include <float.h>
#include <limits.h>
#include <stdlib.h>

#include "kernels.h"

namespace llmk {

constexpr int GEMV_THREADS = 256;
constexpr int GEMV_WAVES = 4;
constexpr int GEMV_MAX_ROWS = 2048;   // input rows one workgroup stages in LDS

__device__ __forceinline__ void store_kv(void* base, int is_bf16, int64_t i, float v) {
  if (is_bf16) static_cast<bf16_t*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// Sum of squares of the K-element input (fp32, or a row of the weight dtype), by one wave. Loads go out
// in groups of 8 per lane with clamped addresses and masked values, so a group is one round trip.
template <typename T>
__device__ __forceinline__ float input_sumsq(const float* inf, const T* inw, int in_is_w, int64_t K, int lane) {
  float ss = 0.0f;
  if (in_is_w && sizeof(T) == 2) {
    const uint4* src = reinterpret_cast<const uint4*>(inw);   // 8 bf16 per 16 B; K % 8 == 0
    const int64_t nv = K / 8;
    for (int64_t b = lane; b < nv; b += 8 * 64) {
      uint4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = src[min(b + k * 64, nv - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float v[8];
        unpack<bf16_t, 8>(t[k], v);
        const float m = (b + k * 64 < nv) ? 1.0f : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(v[e] * m, v[e], ss);
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(in_is_w ? reinterpret_cast<const float*>(inw) : inf);
    const int64_t nv = K / 4;
    for (int64_t b = lane; b < nv; b += 8 * 64) {
      float4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = src[min(b + k * 64, nv - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float m = (b + k * 64 < nv) ? 1.0f : 0.0f;
        ss = fmaf(t[k].x * m, t[k].x, ss);
        ss = fmaf(t[k].y * m, t[k].y, ss);
        ss = fmaf(t[k].z * m, t[k].z, ss);
        ss = fmaf(t[k].w * m, t[k].w, ss);
      }
    }
  }
  return wave_sum(ss);
}

template <typename T, int VEC, int MODE, int LPR>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_t_kernel(const GemvParams p) {
  constexpr int RPI = 64 / LPR;                      // rows covered by one wave load instruction
  constexpr int CB = LPR * VEC;                      // output columns of this workgroup
  constexpr int NACC = (MODE == GM_GATEUP) ? 2 : 1;
  constexpr int U = (MODE == GM_GATEUP) ? 8 : 16;    // load instructions per batch and matrix
  typedef typename Raw<T, VEC>::type RawT;

  __shared__ float x_lds[GEMV_MAX_ROWS];
  __shared__ float red[GEMV_WAVES][NACC][CB];
  __shared__ float fin[NACC][CB];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lc = lane % LPR;                         // column slot of this lane
  const int lr = lane / LPR;                         // row slot of this lane within an instruction
  const int cblk = blockIdx.x % p.n_cblk;
  const int ks = blockIdx.x / p.n_cblk;
  const int64_t col0 = (int64_t)cblk * CB;
  const int64_t k0 = (int64_t)ks * p.rows_per_split;
  const int64_t k1 = min(k0 + p.rows_per_split, p.K);
  const int64_t span = k1 - k0;
  const int64_t per_wave = ((span + GEMV_WAVES - 1) / GEMV_WAVES + RPI - 1) / RPI * RPI;
  const int64_t kw0 = k0 + min(span, (int64_t)wave * per_wave);
  const int64_t kw1 = k0 + min(span, (int64_t)(wave + 1) * per_wave);

  // this lane's columns and the matrix they live in; lanes past N read column 0 (results discarded)
  const int64_t c_raw = col0 + (int64_t)lc * VEC;
  const int64_t c = c_raw < p.N ? c_raw : 0;
  const T* wa = static_cast<const T*>(p.w0);
  const T* wb = static_cast<const T*>(p.w1);
  int64_t lda = p.N;
  if (MODE == GM_QKV) {
    if (c < p.n0) { wa = static_cast<const T*>(p.w0) + c; lda = p.n0; }
    else if (c < p.n0 + p.n1) { wa = static_cast<const T*>(p.w1) + (c - p.n0); lda = p.n1; }
    else { wa = static_cast<const T*>(p.w2) + (c - p.n0 - p.n1); lda = p.N - p.n0 - p.n1; }
  } else {
    wa += c;
    if (MODE == GM_GATEUP) wb += c;
  }

  const int64_t last = max(kw1 - 1, k0);
  constexpr int64_t STEP = (int64_t)U * RPI;   // rows per batch
  // two register sets, A and B, alternate: the next batch is always in flight while one is consumed
  RawT a0[U], a1[U], b0[U], b1[U];
#define LLMK_ISSUE(RA, RB, R)                                         \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                     \
    const int64_t rr = min((R) + u * RPI + lr, last);                 \
    RA[u] = load_raw_stream<T, VEC>(wa + rr * lda);                   \
    if (NACC == 2) RB[u] = load_raw_stream<T, VEC>(wb + rr * lda);    \
  }
  LLMK_ISSUE(a0, b0, kw0)

  // input rows of this workgroup into LDS (RMSNormed when gain is given), zero past k1
  const float* inf = static_cast<const float*>(p.in);
  const T* inw = static_cast<const T*>(p.in);
  if (p.in_state) inw += (int64_t)p.in_state->token * p.K;
  float scale = 1.0f;
  if (p.gain) scale = 1.0f / sqrtf(input_sumsq<T>(inf, inw, p.in_is_w, p.K, lane) / (float)p.K + p.eps);
  const int64_t xr = per_wave * GEMV_WAVES;
  for (int64_t i = threadIdx.x; i < xr; i += GEMV_THREADS) {
    const int64_t row = min(k0 + i, p.K - 1);
    float v = p.in_is_w ? load_elem<T>(inw, row) : inf[row];
    if (p.gain) v = v * scale * p.gain[row];
    x_lds[i] = (k0 + i < k1) ? v : 0.0f;
  }
  __syncthreads();

  float acc[NACC][VEC];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[a][v] = 0.0f;

#define LLMK_CONSUME(RA, RB, R)                                               \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                             \
    const int64_t row = (R) + u * RPI + lr;                                   \
    const float xu = row < kw1 ? x_lds[row - k0] : 0.0f;                      \
    float w[VEC];                                                             \
    unpack<T, VEC>(RA[u], w);                                                 \
    _Pragma("unroll") for (int v = 0; v < VEC; ++v) acc[0][v] = fmaf(w[v], xu, acc[0][v]); \
    if (NACC == 2) {                                                          \
      unpack<T, VEC>(RB[u], w);                                               \
      _Pragma("unroll") for (int v = 0; v < VEC; ++v) acc[NACC - 1][v] = fmaf(w[v], xu, acc[NACC - 1][v]); \
    }                                                                         \
  }

  if (kw1 > kw0) {
    int64_t r = kw0;
    if (r + STEP < kw1) { LLMK_ISSUE(a1, b1, r + STEP) }
    for (;;) {
      LLMK_CONSUME(a0, b0, r)
      r += STEP;
      if (r >= kw1) break;
      if (r + STEP < kw1) { LLMK_ISSUE(a0, b0, r + STEP) }
      LLMK_CONSUME(a1, b1, r)
      r += STEP;
      if (r >= kw1) break;
      if (r + STEP < kw1) { LLMK_ISSUE(a1, b1, r + STEP) }
    }
  }
#undef LLMK_ISSUE
#undef LLMK_CONSUME

  // ---- reduce the row slots of each wave (xor shuffles), then the 4 waves (fixed order) ----
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) acc[a][v] += __shfl_xor(acc[a][v], off, 64);
  if (lr == 0) {
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[wave][a][lc * VEC + v] = acc[a][v];
  }
  __syncthreads();

  if (p.ksplit == 1) {
    for (int j = threadIdx.x; j < CB; j += GEMV_THREADS)
#pragma unroll
      for (int a = 0; a < NACC; ++a) fin[a][j] = ((red[0][a][j] + red[1][a][j]) + red[2][a][j]) + red[3][a][j];
  } else {
    for (int j = threadIdx.x; j < CB; j += GEMV_THREADS) {
      if (col0 + j < p.N) {
#pragma unroll
        for (int a = 0; a < NACC; ++a)
          st_dev(&p.partial[((int64_t)ks * NACC + a) * p.N + col0 + j],
                 ((red[0][a][j] + red[1][a][j]) + red[2][a][j]) + red[3][a][j]);
      }
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (take_ticket(&p.counters[cblk]) == (unsigned)(p.ksplit - 1));
    __syncthreads();
    if (!s_last) return;
    // sum the partials of this strip in split order (all loads of a thread issued together)
    for (int j = threadIdx.x; j < CB * NACC; j += GEMV_THREADS) {
      const int a = j / CB, jj = j % CB;
      float s = 0.0f;
      if (col0 + jj < p.N) {
        const float* src = p.partial + (int64_t)a * p.N + col0 + jj;
        const int64_t stride = (int64_t)NACC * p.N;
        int k = 0;
        for (; k + 16 <= p.ksplit; k += 16) {
          float t[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) t[i] = ld_dev(src + (int64_t)(k + i) * stride);
#pragma unroll
          for (int i = 0; i < 16; ++i) s += t[i];
        }
        for (; k < p.ksplit; ++k) s += ld_dev(src + (int64_t)k * stride);
      }
      fin[a][jj] = s;
    }
    if (threadIdx.x == 0) reset_ticket(&p.counters[cblk]);
  }
  __syncthreads();

  // ---- fused epilogue ----
  for (int j = threadIdx.x; j < CB; j += GEMV_THREADS) {
    const int64_t col = col0 + j;
    if (col >= p.N) continue;
    if (MODE == GM_PLAIN) {
      p.y[col] = fin[0][j];
    } else if (MODE == GM_GATEUP) {
      p.y[col] = silu_f(fin[0][j]) * fin[NACC - 1][j];
    } else if (MODE == GM_RESID) {
      float b;
      if (p.base_is_w) b = load_elem<T>(static_cast<const T*>(p.base) + (int64_t)p.base_state->token * p.N, col);
      else b = p.x[col];
      const float xn = b + fin[0][j];
      p.x[col] = xn;
      if (p.hidden) p.hidden[col] = xn;
    } else {  // GM_QKV: raw q|k|v (rotation and the K/V append happen in the attention kernel)
      p.y[col] = fin[0][j];
    }
  }
}

int gemv_vec(int w_is_bf16, int vec1) { return vec1 ? 1 : (w_is_bf16 ? 8 : 4); }

void gemv_plan(GemvParams& p, int w_is_bf16, int vec1, int target_blocks, int min_cols) {
  const int vec = gemv_vec(w_is_bf16, vec1);
  int lpr = vec1 ? 64 : 16;
  while (lpr < 64 && lpr * vec < min_cols) lpr *= 2;
  p.lpr = lpr;
  const int cb = lpr * vec;
  const int rpi = 64 / lpr;
  p.n_cblk = (int32_t)((p.N + cb - 1) / cb);
  int64_t ksplit = (target_blocks + p.n_cblk / 2) / p.n_cblk;
  if (ksplit < 1) ksplit = 1;
  // a workgroup's rows must fit the LDS input stage (with the per-wave rounding)
  const int64_t max_rows = GEMV_MAX_ROWS - GEMV_WAVES * rpi;
  const int64_t min_split = (p.K + max_rows - 1) / max_rows;
  if (ksplit < min_split) ksplit = min_split;
  if (ksplit > p.K) ksplit = p.K;
  int64_t rps = (p.K + ksplit - 1) / ksplit;
  rps = (rps + GEMV_WAVES * rpi - 1) / (GEMV_WAVES * rpi) * (GEMV_WAVES * rpi);
  if (rps > max_rows) rps = max_rows / (GEMV_WAVES * rpi) * (GEMV_WAVES * rpi);
  p.rows_per_split = rps;
  p.ksplit = (int32_t)((p.K + rps - 1) / rps);
}

template <typename T, int VEC, int MODE, int LPR>
static hipError_t launch_one(const GemvParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemv_t_kernel<T, VEC, MODE, LPR>), dim3((unsigned)(p.n_cblk * p.ksplit)), dim3(GEMV_THREADS), 0,
                     s, p);
  return hipGetLastError();
}

template <typename T, int VEC, int MODE>
static hipError_t launch_lpr(const GemvParams& p, hipStream_t s) {
  switch (p.lpr) {
    case 16: return launch_one<T, VEC, MODE, 16>(p, s);
    case 32: return launch_one<T, VEC, MODE, 32>(p, s);
    case 64: return launch_one<T, VEC, MODE, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t gemv_launch(const GemvParams& p, int mode, int w_is_bf16, int vec1, hipStream_t s) {
  if (vec1) {
    if (mode != GM_PLAIN || p.lpr != 64) return hipErrorInvalidValue;
    return w_is_bf16 ? launch_one<bf16_t, 1, GM_PLAIN, 64>(p, s) : launch_one<float, 1, GM_PLAIN, 64>(p, s);
  }
  if (w_is_bf16) {
    switch (mode) {
      case GM_PLAIN: return launch_lpr<bf16_t, 8, GM_PLAIN>(p, s);
      case GM_QKV: return launch_lpr<bf16_t, 8, GM_QKV>(p, s);
      case GM_RESID: return launch_lpr<bf16_t, 8, GM_RESID>(p, s);
      case GM_GATEUP: return launch_lpr<bf16_t, 8, GM_GATEUP>(p, s);
    }
  } else {
    switch (mode) {
      case GM_PLAIN: return launch_lpr<float, 4, GM_PLAIN>(p, s);
      case GM_QKV: return launch_lpr<float, 4, GM_QKV>(p, s);
      case GM_RESID: return launch_lpr<float, 4, GM_RESID>(p, s);
      case GM_GATEUP: return launch_lpr<float, 4, GM_GATEUP>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

// ================================================================================================
// Output head: row dots + fused argmax
// ================================================================================================

template <typename T, int VEC, int NP, int R>
__global__ __launch_bounds__(GEMV_THREADS) void head_kernel(const HeadParams p) {
  typedef typename Raw<T, VEC>::type RawT;
  __shared__ float s_val[GEMV_WAVES];
  __shared__ int s_idx[GEMV_WAVES];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_block;
  const int64_t r1 = min(r0 + p.rows_per_block, p.rows);
  const T* W = static_cast<const T*>(p.w);

  // rows handled by this wave: groups of R consecutive rows, groups dealt round-robin to the 4 waves.
  // Loads are clamped to the block's last row (a duplicate row is computed and discarded) so every
  // batch is straight-line code: R*NP independent 16-byte loads, then the dots.
  const int64_t last = r1 - 1;
  int64_t rb = r0 + (int64_t)wave * R;
  RawT cur[R][NP];
  auto issue = [&](int64_t base) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int64_t row = min(base + rr, last);
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int64_t cidx = (int64_t)(pp * 64 + lane) * VEC;
        const int64_t cc = cidx < p.cols ? cidx : 0;
        cur[rr][pp] = load_raw_stream<T, VEC>(W + row * p.cols + cc);
      }
    }
  };
  if (rb < r1) issue(rb);

  // input (optionally RMSNormed), held in registers: lane owns columns (pp*64 + lane)*VEC + v
  // (clamped addresses, masked values: no branches between the weight loads and their use)
  float xr[NP][VEC];
  float ss = 0.0f;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int64_t cidx = (int64_t)(pp * 64 + lane) * VEC;
    const bool ok = cidx < p.cols;
    const float4* x4 = reinterpret_cast<const float4*>(p.x + (ok ? cidx : 0));
#pragma unroll
    for (int v4 = 0; v4 < VEC / 4; ++v4) {
      const float4 t = x4[v4];
      xr[pp][v4 * 4 + 0] = ok ? t.x : 0.0f;
      xr[pp][v4 * 4 + 1] = ok ? t.y : 0.0f;
      xr[pp][v4 * 4 + 2] = ok ? t.z : 0.0f;
      xr[pp][v4 * 4 + 3] = ok ? t.w : 0.0f;
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) ss = fmaf(xr[pp][v], xr[pp][v], ss);
  }
  if (p.gain) {
    ss = wave_sum(ss);
    const float sc = 1.0f / sqrtf(ss / (float)p.cols + p.eps);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int64_t cidx = (int64_t)(pp * 64 + lane) * VEC;
      const bool ok = cidx < p.cols;
      const float4* g4 = reinterpret_cast<const float4*>(p.gain + (ok ? cidx : 0));
#pragma unroll
      for (int v4 = 0; v4 < VEC / 4; ++v4) {
        const float4 g = g4[v4];
        xr[pp][v4 * 4 + 0] = xr[pp][v4 * 4 + 0] * sc * g.x;
        xr[pp][v4 * 4 + 1] = xr[pp][v4 * 4 + 1] * sc * g.y;
        xr[pp][v4 * 4 + 2] = xr[pp][v4 * 4 + 2] * sc * g.z;
        xr[pp][v4 * 4 + 3] = xr[pp][v4 * 4 + 3] * sc * g.w;
      }
    }
  }

  float best = -INFINITY;
  int best_i = INT_MAX;
  while (rb < r1) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      float dot = 0.0f;
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        float w[VEC];
        unpack<T, VEC>(cur[rr][pp], w);
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = fmaf(w[v], xr[pp][v], dot);
      }
      dot = wave_sum(dot);
      const int64_t row = rb + rr;
      if (row < r1) {
        if (lane == 0) p.y[row] = dot;
        if (argmax_better(dot, (int)row, best, best_i)) { best = dot; best_i = (int)row; }
      }
    }
    rb += (int64_t)GEMV_WAVES * R;
    if (rb < r1) issue(rb);
  }

  if (!p.part_val) return;

  // ---- argmax pass 1: this workgroup's best ----
  if (lane == 0) { s_val[wave] = best; s_idx[wave] = best_i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = s_val[0];
    int ix = s_idx[0];
    for (int w = 1; w < GEMV_WAVES; ++w)
      if (argmax_better(s_val[w], s_idx[w], v, ix)) { v = s_val[w]; ix = s_idx[w]; }
    st_dev(&p.part_val[blockIdx.x], v);
    st_dev(&p.part_idx[blockIdx.x], ix);
    stores_done();
    s_last = (take_ticket(p.counter) == (unsigned)(gridDim.x - 1));
  }
  __syncthreads();
  if (!s_last) return;

  // ---- pass 2 (last workgroup): best over all workgroups ----
  float v = -INFINITY;
  int ix = INT_MAX;
  for (int b = threadIdx.x; b < (int)gridDim.x; b += GEMV_THREADS) {
    const float bv = ld_dev(&p.part_val[b]);
    const int bi = ld_dev(&p.part_idx[b]);
    if (argmax_better(bv, bi, v, ix)) { v = bv; ix = bi; }
  }
  wave_argmax(v, ix);
  if (lane == 0) { s_val[wave] = v; s_idx[wave] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = s_val[0];
    ix = s_idx[0];
    for (int w = 1; w < GEMV_WAVES; ++w)
      if (argmax_better(s_val[w], s_idx[w], v, ix)) { v = s_val[w]; ix = s_idx[w]; }
    const int step = p.state ? p.state->step : 0;
    p.token_out[step] = ix;
    if (p.logit_out) p.logit_out[step] = v;
    if (p.state) {
      p.state->token = ix;
      p.state->pos = p.state->pos + 1;
      p.state->step = step + 1;
    }
    reset_ticket(p.counter);
  }
}

void head_plan(HeadParams& p, int w_is_bf16) {
  (void)w_is_bf16;
  // about 4 workgroups per CU, each wave handling a few row groups
  int64_t rpb = (p.rows + 1023) / 1024;
  if (rpb < 16) rpb = 16;
  rpb = (rpb + 15) / 16 * 16;
  p.rows_per_block = rpb;
  p.n_blocks = (int32_t)((p.rows + rpb - 1) / rpb);
}

template <typename T, int VEC, int NP, int R>
static hipError_t head_one(const HeadParams& p, hipStream_t s) {
  hipLaunchKernelGGL((head_kernel<T, VEC, NP, R>), dim3((unsigned)p.n_blocks), dim3(GEMV_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t head_dispatch(const HeadParams& p, hipStream_t s) {
  const int64_t np = (p.cols + 64 * VEC - 1) / (64 * VEC);
  if (np <= 1) return head_one<T, VEC, 1, 16>(p, s);
  if (np <= 2) return head_one<T, VEC, 2, 8>(p, s);
  if (np <= 4) return head_one<T, VEC, 4, 4>(p, s);
  if (np <= 8) return head_one<T, VEC, 8, 2>(p, s);
  if (np <= 16) return head_one<T, VEC, 16, 1>(p, s);
  return hipErrorInvalidValue;
}

hipError_t head_launch(const HeadParams& p, int w_is_bf16, hipStream_t s) {
  return w_is_bf16 ? head_dispatch<bf16_t, 8>(p, s) : head_dispatch<float, 4>(p, s);
}

// Fallback for widths that are not a multiple of the vector width: one wave per row, scalar loads.
template <typename T>
__global__ __launch_bounds__(GEMV_THREADS) void rowdot_simple_kernel(const T* W, const float* x, float* y, int64_t rows,
                                                                      int64_t cols) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;
  float s = 0.0f;
  for (int64_t c = lane; c < cols; c += 64) s = fmaf(load_elem<T>(W, row * cols + c), x[c], s);
  s = wave_sum(s);
  if (lane == 0) y[row] = s;
}

hipError_t rowdot_simple_launch(const void* w, int w_is_bf16, const float* x, float* y, int64_t rows, int64_t cols,
                                hipStream_t s) {
  const unsigned grid = (unsigned)((rows + GEMV_WAVES - 1) / GEMV_WAVES);
  if (w_is_bf16)
    hipLaunchKernelGGL(rowdot_simple_kernel<bf16_t>, dim3(grid), dim3(GEMV_THREADS), 0, s,
                       static_cast<const bf16_t*>(w), x, y, rows, cols);
  else
    hipLaunchKernelGGL(rowdot_simple_kernel<float>, dim3(grid), dim3(GEMV_THREADS), 0, s,
                       static_cast<const float*>(w), x, y, rows, cols);
  return hipGetLastError();
}

}  // namespace llmk
