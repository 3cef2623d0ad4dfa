// int8 weights for the decode step on gfx950: a per-group quantizer and the row-dot GEMV over q8 packs.
//
// Format (the library's own: [xpu] "1. CausalLM: the forward path" has decode read packed int8 weights but
// gives no layout):
// each output row of a [rows][K] projection is cut into groups of Q8_GROUP = 128 inputs; a group keeps one
// fp32 scale s = max|w| / 127 and int8 codes q = rint(w / s) (0 for an all-zero group), so w ~ q * s with
// |w - q s| <= s / 2. A pack stores every code of the matrix first, then every scale, both row-major, so a
// row's codes are one contiguous stream of K bytes: 1 + 4/128 bytes per weight against 2 for bf16.
//
// rowdot_q8_kernel has the structure of the bf16 row-dot kernel (a workgroup owns a block of output rows,
// kw waves split K, two register sets of loads alternate, fixed-order reductions, no split-K hand-off), with
// 16-byte loads of 16 codes plus the group's scale. The codes are read as unsigned bytes u = q + 128
// (flip of the top bit, then one byte-to-float conversion each), and a chunk's dot is
//   sum_v q_v x_v = sum_v u_v x_v - 128 * sum_v x_v,
// where the lane computes sum_v x_v of its input slice once per launch.
#include <stdlib.h>

#include "q8.h"

namespace llmk {

constexpr int Q8_THREADS = 256;
constexpr int Q8_WAVES = 4;
constexpr int Q8_V = 16;   // codes per lane per load

// ---- quantizer: one wave per group (two elements a lane) ----------------------------------------------

template <typename T>
__global__ __launch_bounds__(Q8_THREADS) void q8_quantize_kernel(const T* w, int64_t groups, int8_t* codes,
                                                                 float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t first = ((int64_t)blockIdx.x * Q8_THREADS + threadIdx.x) >> 6;
  const int64_t stride = ((int64_t)gridDim.x * Q8_THREADS) >> 6;
  for (int64_t g = first; g < groups; g += stride) {
    // K is a multiple of the group, so group g of the row-major matrix is elements g*128 .. g*128+127
    const int64_t i = g * Q8_GROUP + 2 * lane;
    const float a = load_elem<T>(w, i), b = load_elem<T>(w, i + 1);
    const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
    const float s = __fdiv_rn(amax, 127.0f);
    int qa = 0, qb = 0;
    if (s > 0.0f) {
      qa = (int)rintf(__fdiv_rn(a, s));
      qb = (int)rintf(__fdiv_rn(b, s));
      qa = min(127, max(-127, qa));
      qb = min(127, max(-127, qb));
    }
    const uint16_t pair = (uint16_t)((qa & 0xFF) | ((qb & 0xFF) << 8));
    reinterpret_cast<uint16_t*>(codes + g * Q8_GROUP)[lane] = pair;
    if (lane == 0) scales[g] = s;
  }
}

hipError_t q8_quantize_launch(const void* w, int w_is_bf16, int64_t rows, int64_t K, void* pack, hipStream_t s) {
  const int64_t groups = rows * (K / Q8_GROUP);
  int8_t* codes = static_cast<int8_t*>(pack);
  float* scales = reinterpret_cast<float*>(codes + rows * K);
  const int64_t want = (groups + Q8_WAVES - 1) / Q8_WAVES;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (w_is_bf16)
    hipLaunchKernelGGL(q8_quantize_kernel<bf16_t>, dim3(grid), dim3(Q8_THREADS), 0, s, static_cast<const bf16_t*>(w),
                       groups, codes, scales);
  else
    hipLaunchKernelGGL(q8_quantize_kernel<float>, dim3(grid), dim3(Q8_THREADS), 0, s, static_cast<const float*>(w),
                       groups, codes, scales);
  return hipGetLastError();
}

// ---- row-dot over q8 packs -------------------------------------------------------------------------

__device__ __forceinline__ float ubyte_f(uint32_t w, int j) { return (float)((w >> (8 * j)) & 0xFFu); }

// sum_v u_v x_v over the 16 codes of one load (u = q + 128)
__device__ __forceinline__ float q8_chunk_dot(const uint4& q, const float* x) {
  const uint32_t w[4] = {q.x ^ 0x80808080u, q.y ^ 0x80808080u, q.z ^ 0x80808080u, q.w ^ 0x80808080u};
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t = fmaf(ubyte_f(w[i], j), x[4 * i + j], t);
  return t;
}

template <int NP, int R, int MODE>
__global__ __launch_bounds__(Q8_THREADS) void rowdot_q8_kernel(const RowdotParams p) {
  constexpr int NACC = (MODE == GM_GATEUP) ? 2 : 1;
  __shared__ float part_lds[RD_MAX_ROWS][Q8_WAVES][NACC];
  __shared__ float ss_lds[Q8_WAVES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = p.kw;
  const int groups = Q8_WAVES / kw;
  const int rgi = wave / kw, kseg = wave % kw;
  const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_block;
  const int64_t r1 = min(r0 + p.rows_per_block, p.N);
  const int64_t seg = p.K / kw;                // a multiple of Q8_V
  const int64_t c0 = (int64_t)kseg * seg;
  const int64_t last = r1 - 1;
  const int64_t G = p.K / Q8_GROUP;            // scales per row

  const int8_t* pk0 = static_cast<const int8_t*>(p.w0);
  const int8_t* pk1 = static_cast<const int8_t*>(p.w1);
  const int8_t* pk2 = static_cast<const int8_t*>(p.w2);
  // pack and row within it of output row R_ (matrix M_ of the gate|up pair)
#define Q8_PACK(R_, M_)                                                                                  \
  (MODE == GM_QKV ? ((R_) < p.n0 ? pk0 : (R_) < p.n0 + p.n1 ? pk1 : pk2) : ((M_) == 0 ? pk0 : pk1))
#define Q8_LOCAL(R_) (MODE == GM_QKV ? ((R_) < p.n0 ? (R_) : (R_) < p.n0 + p.n1 ? (R_) - p.n0 : (R_) - p.n0 - p.n1) : (R_))
#define Q8_ROWS(R_) (MODE == GM_QKV ? ((R_) < p.n0 ? p.n0 : (R_) < p.n0 + p.n1 ? p.n1 : p.N - p.n0 - p.n1) : p.N)

  uint4 a0[NACC][R][NP], a1[NACC][R][NP];
  float s0[NACC][R][NP], s1[NACC][R][NP];
#define Q8_ISSUE(BUF, SB, RB)                                                                         \
  _Pragma("unroll") for (int rr = 0; rr < R; ++rr) {                                                  \
    const int64_t row = min((RB) + rr, last);                                                         \
    const int64_t lr = Q8_LOCAL(row);                                                                 \
    const int64_t nr = Q8_ROWS(row);                                                                  \
    _Pragma("unroll") for (int m = 0; m < NACC; ++m) {                                                \
      const int8_t* pk = Q8_PACK(row, m);                                                             \
      const int8_t* cw = pk + lr * p.K;                                                               \
      const float* sw = reinterpret_cast<const float*>(pk + nr * p.K) + lr * G;                       \
      _Pragma("unroll") for (int pp = 0; pp < NP; ++pp) {                                             \
        const int64_t cc = (int64_t)(pp * 64 + lane) * Q8_V;                                          \
        const int64_t col = c0 + (cc < seg ? cc : 0);                                                 \
        BUF[m][rr][pp] = gload_stream(cw + col);                                                      \
        SB[m][rr][pp] = sw[col / Q8_GROUP];                                                           \
      }                                                                                               \
    }                                                                                                 \
  }

  const int64_t step = (int64_t)groups * R;
  int64_t rb = r0 + (int64_t)rgi * R;
  if (rb < r1) { Q8_ISSUE(a0, s0, rb) }

  // this lane's input slices: fp32, or the bf16 embedding row chosen by the device-side token
  const float* inf = static_cast<const float*>(p.in);
  const bf16_t* inw = static_cast<const bf16_t*>(p.in);
  if (p.in_state) inw += (int64_t)p.in_state->token * p.K;
  float xr[NP][Q8_V];
  float xs[NP];
  float ss = 0.0f;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int64_t cc = (int64_t)(pp * 64 + lane) * Q8_V;
    const bool ok = cc < seg;
    const int64_t col = c0 + (ok ? cc : 0);
    float t[Q8_V];
    if (p.in_is_w) {
      unpack<bf16_t, 8>(load_raw<bf16_t, 8>(inw + col), t);
      unpack<bf16_t, 8>(load_raw<bf16_t, 8>(inw + col + 8), t + 8);
    } else {
#pragma unroll
      for (int v4 = 0; v4 < Q8_V / 4; ++v4) {
        const float4 f = reinterpret_cast<const float4*>(inf + col)[v4];
        t[v4 * 4 + 0] = f.x; t[v4 * 4 + 1] = f.y; t[v4 * 4 + 2] = f.z; t[v4 * 4 + 3] = f.w;
      }
    }
#pragma unroll
    for (int v = 0; v < Q8_V; ++v) {
      xr[pp][v] = ok ? t[v] : 0.0f;
      ss = fmaf(xr[pp][v], xr[pp][v], ss);
    }
    if (p.gain) {
#pragma unroll
      for (int v4 = 0; v4 < Q8_V / 4; ++v4) {
        const float4 g = reinterpret_cast<const float4*>(p.gain + col)[v4];
        xr[pp][v4 * 4 + 0] *= g.x; xr[pp][v4 * 4 + 1] *= g.y; xr[pp][v4 * 4 + 2] *= g.z; xr[pp][v4 * 4 + 3] *= g.w;
      }
    }
    float sx = 0.0f;
#pragma unroll
    for (int v = 0; v < Q8_V; ++v) sx += xr[pp][v];
    xs[pp] = 128.0f * sx;
  }
  if (p.gain) {
    ss = wave_sum(ss);
    if (rgi == 0 && lane == 0) ss_lds[kseg] = ss;
  }

  // The R x NACC dots of a batch reduce across the wave together: each halving step trades half of a lane's
  // values with the partner lane, so M values take M - 1 + log2(64 / M) shuffles instead of 6 M; lane l ends
  // with the total of value j(l) = sum over steps of (l & o ? h : 0), held by the lanes l % (64 / M) == 0.
  constexpr int M = R * NACC;
  constexpr int SPAN = 64 / M;
#define Q8_CONSUME(BUF, SB, RB)                                                                       \
  {                                                                                                   \
    float v[M];                                                                                       \
    _Pragma("unroll") for (int rr = 0; rr < R; ++rr) {                                                \
      _Pragma("unroll") for (int m = 0; m < NACC; ++m) {                                              \
        float dot = 0.0f;                                                                             \
        _Pragma("unroll") for (int pp = 0; pp < NP; ++pp)                                             \
          dot = fmaf(SB[m][rr][pp], q8_chunk_dot(BUF[m][rr][pp], xr[pp]) - xs[pp], dot);              \
        v[rr * NACC + m] = dot;                                                                       \
      }                                                                                               \
    }                                                                                                 \
    int j = 0;                                                                                        \
    _Pragma("unroll") for (int h = M / 2, o = 32; h >= 1; h /= 2, o /= 2) {                           \
      const bool upper = (lane & o) != 0;                                                             \
      j += upper ? h : 0;                                                                             \
      _Pragma("unroll") for (int i = 0; i < h; ++i) {                                                 \
        const float send = upper ? v[i] : v[i + h];                                                   \
        const float keep = upper ? v[i + h] : v[i];                                                   \
        v[i] = keep + __shfl_xor(send, o, 64);                                                        \
      }                                                                                               \
    }                                                                                                 \
    _Pragma("unroll") for (int o = SPAN / 2; o >= 1; o /= 2) v[0] += __shfl_xor(v[0], o, 64);         \
    const int64_t row = (RB) + j / NACC;                                                              \
    if ((lane & (SPAN - 1)) == 0 && row < r1) part_lds[row - r0][kseg][j % NACC] = v[0];              \
  }

  if (rb < r1) {
    if (rb + step < r1) { Q8_ISSUE(a1, s1, rb + step) }
    for (;;) {
      Q8_CONSUME(a0, s0, rb)
      rb += step;
      if (rb >= r1) break;
      if (rb + step < r1) { Q8_ISSUE(a0, s0, rb + step) }
      Q8_CONSUME(a1, s1, rb)
      rb += step;
      if (rb >= r1) break;
      if (rb + step < r1) { Q8_ISSUE(a1, s1, rb + step) }
    }
  }
#undef Q8_ISSUE
#undef Q8_CONSUME
#undef Q8_PACK
#undef Q8_LOCAL
#undef Q8_ROWS
  __syncthreads();

  // ---- epilogue: one thread per row, segments summed in order ----
  float scale = 1.0f;
  if (p.gain) {
    float tot = ss_lds[0];
    for (int k = 1; k < kw; ++k) tot += ss_lds[k];
    scale = 1.0f / sqrtf(tot / (float)p.K + p.eps);
  }
  for (int64_t row = r0 + threadIdx.x; row < r1; row += Q8_THREADS) {
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
      if (p.base_is_w) b = load_elem<bf16_t>(static_cast<const bf16_t*>(p.base) + (int64_t)p.base_state->token * p.N, row);
      else b = p.x[row];
      const float xn = b + acc[0];
      p.x[row] = xn;
      if (p.hidden) p.hidden[row] = xn;
    }
  }
}

int rowdot_q8_plan(RowdotParams& p, int mode) {
  if (p.K % Q8_GROUP != 0) return -1;
  // as many segment waves as keep a segment at one full load per lane (1,024 codes) or more
  int kw = 4;
  while (kw > 1 && p.K / kw < 64 * Q8_V) kw /= 2;
  const int64_t seg = p.K / kw;
  const int np = (int)((seg + 64 * Q8_V - 1) / (64 * Q8_V));
  if (np > 4) return -1;
  p.kw = kw;
  p.np = np <= 1 ? 1 : np <= 2 ? 2 : 4;
  int r = p.np == 1 ? 8 : p.np == 2 ? 4 : 2;
  if (mode == GM_GATEUP) r /= 2;
  p.r = r;
  const int64_t quantum = (int64_t)(Q8_WAVES / kw) * r;
  // workgroups per launch, measured on the Llama-3-8B shape: 512 for gate|up and the down projection (longer
  // rows per workgroup amortise its prologue), 2,048 for the vocabulary-wide head, 1,024 for q|k|v and o
  const int64_t dflt = (mode == GM_GATEUP || (mode == GM_RESID && p.K > p.N)) ? 512 : mode == GM_PLAIN ? 2048 : 1024;
  const int64_t target = dflt;
  int64_t rpb = (p.N + target - 1) / target;
  rpb = (rpb + quantum - 1) / quantum * quantum;
  if (rpb > RD_MAX_ROWS) rpb = RD_MAX_ROWS / quantum * quantum;
  p.rows_per_block = rpb;
  p.n_blocks = (int32_t)((p.N + rpb - 1) / rpb);
  return 0;
}

template <int NP, int R, int MODE>
static hipError_t q8_one(const RowdotParams& p, hipStream_t s) {
  hipLaunchKernelGGL((rowdot_q8_kernel<NP, R, MODE>), dim3((unsigned)p.n_blocks), dim3(Q8_THREADS), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
static hipError_t q8_np(const RowdotParams& p, hipStream_t s) {
  constexpr int G = (MODE == GM_GATEUP) ? 2 : 1;
  const bool x2 = p.r == 2 * ((p.np == 1 ? 8 : p.np == 2 ? 4 : 2) / G);
  switch (p.np) {
    case 1: return x2 ? q8_one<1, 16 / G, MODE>(p, s) : q8_one<1, 8 / G, MODE>(p, s);
    case 2: return x2 ? q8_one<2, 8 / G, MODE>(p, s) : q8_one<2, 4 / G, MODE>(p, s);
    case 4: return x2 ? q8_one<4, 4 / G, MODE>(p, s) : q8_one<4, 2 / G, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t rowdot_q8_launch(const RowdotParams& p, int mode, hipStream_t s) {
  switch (mode) {
    case GM_PLAIN: return q8_np<GM_PLAIN>(p, s);
    case GM_QKV: return q8_np<GM_QKV>(p, s);
    case GM_RESID: return q8_np<GM_RESID>(p, s);
    case GM_GATEUP: return q8_np<GM_GATEUP>(p, s);
  }
  return hipErrorInvalidValue;
}

// ---- decode state after a greedy head ------------------------------------------------------------

__global__ void state_advance_kernel(DecodeState* st, const int32_t* tok, int32_t* token_out) {
  if (threadIdx.x != 0) return;
  const int32_t step = st->step;
  const int32_t t = *tok;
  token_out[step] = t;
  st->token = t;
  st->pos = st->pos + 1;
  st->step = step + 1;
}

hipError_t state_advance_launch(DecodeState* st, const int32_t* tok, int32_t* token_out, hipStream_t s) {
  hipLaunchKernelGGL(state_advance_kernel, dim3(1), dim3(64), 0, s, st, tok, token_out);
  return hipGetLastError();
}

}  // namespace llmk
