// Row-dot GEMV for gfx950: y[r] = W[r] . h with W [rows][K] row-major (weights stored output-major),
// the layout in which every projection of the decode step streams contiguous rows.
//
//   - A workgroup (4 waves) owns a contiguous block of output rows. kw waves (1, 2 or 4) share a row and
//     split K into kw contiguous segments; each lane holds its VEC-wide slices of the input segment in
//     registers and streams R rows at a time with 16-byte loads (NP loads per row), two register sets
//     alternating so the next rows are in flight while the current ones are summed.
//   - Dots reduce within the wave (xor shuffles) and across the kw segment waves through LDS in a fixed
//     order; nothing crosses workgroups, so there is no split-K hand-off and no tail.
//   - The input is fp32 or the embedding row (weight dtype, chosen by the device-side token), optionally
//     RMSNormed: the lanes already hold x, so the fp32 square sum is free, and since the norm scale is one
//     scalar per step it multiplies the finished dots (y = scale * W (x * g)).
//   - Epilogues per row: plain store (also the stacked q|k|v rows), residual add x = base + y (base may be
//     the embedding row) with an optional copy of x, and SiLU-gate u = silu(gate . h) * (up . h) where
//     the same lanes stream row r of gate and of up.
#include <stdlib.h>

#include "kernels.h"

namespace llmk {

constexpr int RD_THREADS = 256;
constexpr int RD_WAVES = 4;

// MODE: GM_PLAIN (one matrix), GM_QKV (q|k|v rows stacked from three matrices), GM_RESID, GM_GATEUP.
// With an RMSNorm input, y = scale * sum_k W[r][k] (x[k] g[k]): the scale is a per-step scalar, applied
// after the dot, and its square sum comes from the slices the segment waves already hold.
template <typename T, int VEC, int NP, int R, int MODE>
__global__ __launch_bounds__(RD_THREADS) void rowdot_kernel(const RowdotParams p) {
  constexpr int NACC = (MODE == GM_GATEUP) ? 2 : 1;
  typedef typename Raw<T, VEC>::type RawT;
  __shared__ float part_lds[RD_MAX_ROWS][4][NACC];
  __shared__ float ss_lds[4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = p.kw;
  const int groups = RD_WAVES / kw;            // row groups per workgroup
  const int rgi = wave / kw, kseg = wave % kw;
  const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_block;
  const int64_t r1 = min(r0 + p.rows_per_block, p.N);
  const int64_t seg = p.K / kw;                // K is a multiple of kw * VEC
  const int64_t c0 = (int64_t)kseg * seg;
  const int64_t last = r1 - 1;

  const T* wbase0 = static_cast<const T*>(p.w0);
  const T* wbase1 = static_cast<const T*>(p.w1);
  const T* wbase2 = static_cast<const T*>(p.w2);
#define LLMK_ROW_PTR(R_, M_)                                                                           \
  (MODE == GM_QKV ? ((R_) < p.n0 ? wbase0 + (R_) * p.K                                                  \
                     : (R_) < p.n0 + p.n1 ? wbase1 + ((R_) - p.n0) * p.K                                 \
                     : wbase2 + ((R_) - p.n0 - p.n1) * p.K)                                              \
                  : ((M_) == 0 ? wbase0 : wbase1) + (R_) * p.K)

  RawT a0[NACC][R][NP], a1[NACC][R][NP];
#define LLMK_RD_ISSUE(BUF, RB)                                                         \
  _Pragma("unroll") for (int rr = 0; rr < R; ++rr) {                                   \
    const int64_t row = min((RB) + rr, last);                                          \
    _Pragma("unroll") for (int m = 0; m < NACC; ++m) {                                 \
      const T* base = LLMK_ROW_PTR(row, m) + c0;                                       \
      _Pragma("unroll") for (int pp = 0; pp < NP; ++pp) {                              \
        const int64_t cc = (int64_t)(pp * 64 + lane) * VEC;                            \
        BUF[m][rr][pp] = load_raw_stream<T, VEC>(base + (cc < seg ? cc : 0));          \
      }                                                                                \
    }                                                                                  \
  }

  const int64_t step = (int64_t)groups * R;
  int64_t rb = r0 + (int64_t)rgi * R;
  if (rb < r1) { LLMK_RD_ISSUE(a0, rb) }

  // this lane's input slices (vector loads), their square sum, then x * gain
  const float* inf = static_cast<const float*>(p.in);
  const T* inw = static_cast<const T*>(p.in);
  if (p.in_state) inw += (int64_t)p.in_state->token * p.K;
  float xr[NP][VEC];
  float ss = 0.0f;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int64_t cc = (int64_t)(pp * 64 + lane) * VEC;
    const bool ok = cc < seg;
    const int64_t col = c0 + (ok ? cc : 0);
    float t[VEC];
    if (p.in_is_w) {
      unpack<T, VEC>(load_raw<T, VEC>(inw + col), t);
    } else {
#pragma unroll
      for (int v4 = 0; v4 < VEC / 4; ++v4) {
        const float4 f = reinterpret_cast<const float4*>(inf + col)[v4];
        t[v4 * 4 + 0] = f.x; t[v4 * 4 + 1] = f.y; t[v4 * 4 + 2] = f.z; t[v4 * 4 + 3] = f.w;
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      xr[pp][v] = ok ? t[v] : 0.0f;
      ss = fmaf(xr[pp][v], xr[pp][v], ss);
    }
    if (p.gain) {
#pragma unroll
      for (int v4 = 0; v4 < VEC / 4; ++v4) {
        const float4 g = reinterpret_cast<const float4*>(p.gain + col)[v4];
        xr[pp][v4 * 4 + 0] *= g.x; xr[pp][v4 * 4 + 1] *= g.y; xr[pp][v4 * 4 + 2] *= g.z; xr[pp][v4 * 4 + 3] *= g.w;
      }
    }
  }
  if (p.gain) {
    ss = wave_sum(ss);
    if (rgi == 0 && lane == 0) ss_lds[kseg] = ss;
  }

#define LLMK_RD_CONSUME(BUF, RB)                                                       \
  _Pragma("unroll") for (int rr = 0; rr < R; ++rr) {                                   \
    _Pragma("unroll") for (int m = 0; m < NACC; ++m) {                                 \
      float dot = 0.0f;                                                                \
      _Pragma("unroll") for (int pp = 0; pp < NP; ++pp) {                              \
        float w[VEC];                                                                  \
        unpack<T, VEC>(BUF[m][rr][pp], w);                                             \
        _Pragma("unroll") for (int v = 0; v < VEC; ++v) dot = fmaf(w[v], xr[pp][v], dot); \
      }                                                                                \
      dot = wave_sum(dot);                                                             \
      const int64_t row = (RB) + rr;                                                   \
      if (lane == 0 && row < r1) part_lds[row - r0][kseg][m] = dot;                    \
    }                                                                                  \
  }

  if (rb < r1) {
    if (rb + step < r1) { LLMK_RD_ISSUE(a1, rb + step) }
    for (;;) {
      LLMK_RD_CONSUME(a0, rb)
      rb += step;
      if (rb >= r1) break;
      if (rb + step < r1) { LLMK_RD_ISSUE(a0, rb + step) }
      LLMK_RD_CONSUME(a1, rb)
      rb += step;
      if (rb >= r1) break;
      if (rb + step < r1) { LLMK_RD_ISSUE(a1, rb + step) }
    }
  }
#undef LLMK_RD_ISSUE
#undef LLMK_RD_CONSUME
#undef LLMK_ROW_PTR
  __syncthreads();

  // ---- epilogue: one thread per row, segments summed in order ----
  float scale = 1.0f;
  if (p.gain) {
    float tot = ss_lds[0];
    for (int k = 1; k < kw; ++k) tot += ss_lds[k];
    scale = 1.0f / sqrtf(tot / (float)p.K + p.eps);
  }
  for (int64_t row = r0 + threadIdx.x; row < r1; row += RD_THREADS) {
    float acc[NACC];
#pragma unroll
    for (int m = 0; m < NACC; ++m) {
      float s = part_lds[row - r0][0][m];
      for (int k = 1; k < kw; ++k) s += part_lds[row - r0][k][m];
      acc[m] = s * scale;
    }
    if (MODE == GM_PLAIN || MODE == GM_QKV) {
      p.y[row] = acc[0];
    } else if (MODE == GM_GATEUP) {
      p.y[row] = silu_f(acc[0]) * acc[NACC - 1];
    } else {  // GM_RESID
      float b;
      if (p.base_is_w) b = load_elem<T>(static_cast<const T*>(p.base) + (int64_t)p.base_state->token * p.N, row);
      else b = p.x[row];
      const float xn = b + acc[0];
      p.x[row] = xn;
      if (p.hidden) p.hidden[row] = xn;
    }
  }
}

// ------------------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------------------

int rowdot_plan(RowdotParams& p, int w_is_bf16, int mode) {
  const int vec = w_is_bf16 ? 8 : 4;
  if (p.K % vec != 0) return -1;
  // split K over as many of the 4 waves as the vector width allows: each wave holds a quarter of x
  int kw = 4;
  while (kw > 1 && (p.K % kw != 0 || (p.K / kw) % vec != 0)) kw /= 2;
  if (p.K % kw != 0 || (p.K / kw) % vec != 0) return -1;
  const int np = (int)((p.K / kw + 64 * vec - 1) / (64 * vec));
  if (np > 8) return -1;
  p.kw = kw;
  p.np = np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
  int r = p.np == 1 ? 8 : p.np == 2 ? 4 : p.np == 4 ? 2 : 1;   // about 8 loads per row batch
  if (mode == GM_GATEUP) r = r > 1 ? r / 2 : 1;
  p.r = r;
  const int64_t quantum = (int64_t)(RD_WAVES / kw) * p.r;
  const int64_t target = 1024;   // workgroups per launch
  int64_t rpb = (p.N + target - 1) / target;
  rpb = (rpb + quantum - 1) / quantum * quantum;
  if (rpb > RD_MAX_ROWS) rpb = RD_MAX_ROWS / quantum * quantum;
  p.rows_per_block = rpb;
  p.n_blocks = (int32_t)((p.N + rpb - 1) / rpb);
  return 0;
}

template <typename T, int VEC, int NP, int R, int MODE>
static hipError_t rd_one(const RowdotParams& p, hipStream_t s) {
  hipLaunchKernelGGL((rowdot_kernel<T, VEC, NP, R, MODE>), dim3((unsigned)p.n_blocks), dim3(RD_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename T, int VEC, int MODE>
static hipError_t rd_np(const RowdotParams& p, hipStream_t s) {
  constexpr int G = (MODE == GM_GATEUP) ? 2 : 1;   // gate|up streams two rows per row slot
  switch (p.np) {
    case 1: return rd_one<T, VEC, 1, 8 / G, MODE>(p, s);
    case 2: return rd_one<T, VEC, 2, 4 / G, MODE>(p, s);
    case 4: return rd_one<T, VEC, 4, 2 / G, MODE>(p, s);
    case 8: return rd_one<T, VEC, 8, 1, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t rowdot_launch(const RowdotParams& p, int mode, int w_is_bf16, hipStream_t s) {
  if (w_is_bf16) {
    switch (mode) {
      case GM_PLAIN: return rd_np<bf16_t, 8, GM_PLAIN>(p, s);
      case GM_QKV: return rd_np<bf16_t, 8, GM_QKV>(p, s);
      case GM_RESID: return rd_np<bf16_t, 8, GM_RESID>(p, s);
      case GM_GATEUP: return rd_np<bf16_t, 8, GM_GATEUP>(p, s);
    }
  } else {
    switch (mode) {
      case GM_PLAIN: return rd_np<float, 4, GM_PLAIN>(p, s);
      case GM_QKV: return rd_np<float, 4, GM_QKV>(p, s);
      case GM_RESID: return rd_np<float, 4, GM_RESID>(p, s);
      case GM_GATEUP: return rd_np<float, 4, GM_GATEUP>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------------------
// transpose: dst[c][r] = src[r][c] (one-time repacking of weights into the output-major layout)
// ------------------------------------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, T* dst, int64_t rows, int64_t cols) {
  __shared__ T tile[64][65];
  const int64_t br = (int64_t)blockIdx.y * 64, bc = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = br + i, c = bc + tx;
    if (r < rows && c < cols) tile[i][tx] = src[r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = bc + i, r = br + tx;
    if (r < rows && c < cols) dst[c * rows + r] = tile[tx][i];
  }
}

hipError_t transpose_launch(const void* src, void* dst, int64_t rows, int64_t cols, int is_bf16, hipStream_t s) {
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  if (is_bf16)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(src),
                       static_cast<bf16_t*>(dst), rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
                       static_cast<float*>(dst), rows, cols);
  return hipGetLastError();
}

}  // namespace llmk
