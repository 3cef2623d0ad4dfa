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

#include "kernels.h"

namespace llmk {

constexpr int GEMV_THREADS = 256;
constexpr int GEMV_WAVES = 4;

__device__ __forceinline__ void store_kv(void* base, int is_bf16, int64_t i, float v) {
  if (is_bf16) static_cast<bf16_t*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

template <typename T, int VEC, int MODE>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_t_kernel(const GemvParams p) {
  constexpr int CB = 64 * VEC;
  constexpr int NACC = (MODE == GM_GATEUP) ? 2 : 1;
  constexpr int U = (MODE == GM_GATEUP) ? 4 : 8;   // rows per load batch (divides 64)
  typedef typename Raw<T, VEC>::type RawT;

  __shared__ float red[GEMV_WAVES][NACC][CB];
  __shared__ float fin[NACC][CB];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cblk = blockIdx.x % p.n_cblk;
  const int ks = blockIdx.x / p.n_cblk;
  const int64_t col0 = (int64_t)cblk * CB;
  const int64_t k0 = (int64_t)ks * p.rows_per_split;
  const int64_t k1 = min(k0 + p.rows_per_split, p.K);
  const int64_t span = k1 - k0;
  const int64_t per_wave = ((span + GEMV_WAVES - 1) / GEMV_WAVES + U - 1) / U * U;
  const int64_t kw0 = k0 + min(span, (int64_t)wave * per_wave);
  const int64_t kw1 = k0 + min(span, (int64_t)(wave + 1) * per_wave);

  // this lane's columns and the matrix they live in
  const int64_t c = col0 + (int64_t)lane * VEC;
  const bool active = c < p.N;
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

  RawT ca[U], cb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = kw0 + u;
    if (active && r < kw1) {
      ca[u] = load_raw<T, VEC>(wa + r * lda);
      if (NACC == 2) cb[u] = load_raw<T, VEC>(wb + r * lda);
    } else {
      ca[u] = RawT{};
      cb[u] = RawT{};
    }
  }

  // ---- prologue: the input vector (optionally RMSNormed), overlapping the first loads ----
  const float* inf = static_cast<const float*>(p.in);
  const T* inw = static_cast<const T*>(p.in);
  if (p.in_state) inw += (int64_t)p.in_state->token * p.K;
  float scale = 1.0f;
  if (p.gain) {
    float ss = 0.0f;
#pragma unroll 8
    for (int64_t i = lane; i < p.K; i += 64) {
      const float v = p.in_is_w ? load_elem<T>(inw, i) : inf[i];
      ss += v * v;
    }
    ss = wave_sum(ss);
    scale = 1.0f / sqrtf(ss / (float)p.K + p.eps);
  }

  float acc[NACC][VEC];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[a][v] = 0.0f;

  float xseg = 0.0f;
  for (int64_t r = kw0; r < kw1; r += U) {
    const int seg_lane = (int)((r - kw0) & 63);
    if (seg_lane == 0) {
      const int64_t rr = r + lane;
      float v = 0.0f;
      if (rr < kw1) {
        v = p.in_is_w ? load_elem<T>(inw, rr) : inf[rr];
        if (p.gain) v = v * scale * p.gain[rr];
      }
      xseg = v;
    }
    RawT na[U], nb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rn = r + U + u;
      if (active && rn < kw1) {
        na[u] = load_raw<T, VEC>(wa + rn * lda);
        if (NACC == 2) nb[u] = load_raw<T, VEC>(wb + rn * lda);
      } else {
        na[u] = RawT{};
        nb[u] = RawT{};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float xv = readlane_f(xseg, seg_lane + u);
      float w[VEC];
      unpack<T, VEC>(ca[u], w);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[0][v] = fmaf(w[v], xv, acc[0][v]);
      if (NACC == 2) {
        unpack<T, VEC>(cb[u], w);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[NACC - 1][v] = fmaf(w[v], xv, acc[NACC - 1][v]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ca[u] = na[u];
      cb[u] = nb[u];
    }
  }

  // ---- reduce the 4 waves (fixed order) ----
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wave][a][lane * VEC + v] = acc[a][v];
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
          p.partial[((int64_t)ks * NACC + a) * p.N + col0 + j] =
              ((red[0][a][j] + red[1][a][j]) + red[2][a][j]) + red[3][a][j];
      }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev = atomicAdd(&p.counters[cblk], 1u);
      s_last = (prev == (unsigned)(p.ksplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // sum the partials of this strip in split order; P threads share a column group
    if constexpr (VEC >= 4) {
      constexpr int NG = CB / 4;                  // float4 column groups
      constexpr int P = GEMV_THREADS / NG;        // split ranges per group (2 for bf16, 4 for fp32)
      float4* tmp = reinterpret_cast<float4*>(&red[0][0][0]);   // reuse: [NACC][P][NG] float4
      const int g = threadIdx.x % NG, part = threadIdx.x / NG;
      const int per = (p.ksplit + P - 1) / P;
      const int kb = part * per, ke = min(p.ksplit, kb + per);
      const int64_t col = col0 + (int64_t)g * 4;
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        if (col < p.N) {
          int k = kb;
          for (; k + 8 <= ke; k += 8) {
            float4 t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              t[i] = *reinterpret_cast<const float4*>(p.partial + ((int64_t)(k + i) * NACC + a) * p.N + col);
#pragma unroll
            for (int i = 0; i < 8; ++i) { s.x += t[i].x; s.y += t[i].y; s.z += t[i].z; s.w += t[i].w; }
          }
          for (; k < ke; ++k) {
            const float4 t = *reinterpret_cast<const float4*>(p.partial + ((int64_t)k * NACC + a) * p.N + col);
            s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
          }
        }
        tmp[(a * P + part) * NG + g] = s;
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          float4 s = tmp[(a * P) * NG + g];
          for (int q = 1; q < P; ++q) {
            const float4 t = tmp[(a * P + q) * NG + g];
            s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
          }
          fin[a][g * 4 + 0] = s.x; fin[a][g * 4 + 1] = s.y; fin[a][g * 4 + 2] = s.z; fin[a][g * 4 + 3] = s.w;
        }
      }
    } else {
      for (int j = threadIdx.x; j < CB; j += GEMV_THREADS) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          float s = 0.0f;
          if (col0 + j < p.N)
            for (int k = 0; k < p.ksplit; ++k) s += p.partial[((int64_t)k * NACC + a) * p.N + col0 + j];
          fin[a][j] = s;
        }
      }
    }
    if (threadIdx.x == 0) p.counters[cblk] = 0u;
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
    } else {  // GM_QKV
      const int hd = p.head_dim, half = hd >> 1;
      const int i = (int)(col % hd);
      const int pos = p.state->pos;
      const bool is_q = col < p.n0;
      const bool is_k = !is_q && col < p.n0 + p.n1;
      float val = fin[0][j];
      if (is_q || is_k) {
        bool first;
        int jj, partner;
        if (p.rope_layout == 0) {
          first = i < half;
          jj = first ? i : i - half;
          partner = first ? j + half : j - half;
        } else {
          first = (i & 1) == 0;
          jj = i >> 1;
          partner = j ^ 1;
        }
        const float cs = p.rope_table[((int64_t)pos * half + jj) * 2 + 0];
        const float sn = p.rope_table[((int64_t)pos * half + jj) * 2 + 1];
        const float other = fin[0][partner];
        val = first ? (val * cs - other * sn) : (other * sn + val * cs);
      }
      if (is_q) p.y[col] = val;
      else if (is_k) store_kv(p.kcache, p.kv_is_bf16, p.kv_off + (int64_t)pos * p.n1 + (col - p.n0), val);
      else store_kv(p.vcache, p.kv_is_bf16, p.kv_off + (int64_t)pos * p.n1 + (col - p.n0 - p.n1), val);
    }
  }
}

void gemv_plan(GemvParams& p, int w_is_bf16, int vec1, int target_blocks, int min_rows) {
  const int cb = gemv_cols_per_block(w_is_bf16, vec1);
  p.n_cblk = (int32_t)((p.N + cb - 1) / cb);
  int64_t want = target_blocks / p.n_cblk;
  if (want < 1) want = 1;
  int64_t rps = (p.K + want - 1) / want;
  if (rps < min_rows) rps = min_rows;
  rps = (rps + 31) / 32 * 32;
  if (rps >= p.K) rps = p.K;
  p.rows_per_split = rps;
  p.ksplit = (int32_t)((p.K + rps - 1) / rps);
}

template <typename T, int VEC, int MODE>
static hipError_t launch_one(const GemvParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemv_t_kernel<T, VEC, MODE>), dim3((unsigned)(p.n_cblk * p.ksplit)), dim3(GEMV_THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t gemv_launch(const GemvParams& p, int mode, int w_is_bf16, int vec1, hipStream_t s) {
  if (vec1) {
    if (mode != GM_PLAIN) return hipErrorInvalidValue;
    return w_is_bf16 ? launch_one<bf16_t, 1, GM_PLAIN>(p, s) : launch_one<float, 1, GM_PLAIN>(p, s);
  }
  if (w_is_bf16) {
    switch (mode) {
      case GM_PLAIN: return launch_one<bf16_t, 8, GM_PLAIN>(p, s);
      case GM_QKV: return launch_one<bf16_t, 8, GM_QKV>(p, s);
      case GM_RESID: return launch_one<bf16_t, 8, GM_RESID>(p, s);
      case GM_GATEUP: return launch_one<bf16_t, 8, GM_GATEUP>(p, s);
    }
  } else {
    switch (mode) {
      case GM_PLAIN: return launch_one<float, 4, GM_PLAIN>(p, s);
      case GM_QKV: return launch_one<float, 4, GM_QKV>(p, s);
      case GM_RESID: return launch_one<float, 4, GM_RESID>(p, s);
      case GM_GATEUP: return launch_one<float, 4, GM_GATEUP>(p, s);
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

  // rows handled by this wave: groups of R consecutive rows, groups dealt round-robin to the 4 waves
  int64_t rb = r0 + (int64_t)wave * R;
  RawT cur[R][NP];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int64_t c = (int64_t)(pp * 64 + lane) * VEC;
      if (rb + rr < r1 && c < p.cols) cur[rr][pp] = load_raw<T, VEC>(W + (rb + rr) * p.cols + c);
      else cur[rr][pp] = RawT{};
    }

  // input (optionally RMSNormed), held in registers: lane owns columns (pp*64 + lane)*VEC + v
  float xr[NP][VEC];
  float ss = 0.0f;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int64_t c = (int64_t)(pp * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      xr[pp][v] = (c + v < p.cols) ? p.x[c + v] : 0.0f;
      ss += xr[pp][v] * xr[pp][v];
    }
  }
  if (p.gain) {
    ss = wave_sum(ss);
    const float sc = 1.0f / sqrtf(ss / (float)p.cols + p.eps);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int64_t c = (int64_t)(pp * 64 + lane) * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) xr[pp][v] = (c + v < p.cols) ? xr[pp][v] * sc * p.gain[c + v] : 0.0f;
    }
  }

  float best = -INFINITY;
  int best_i = INT_MAX;
  for (; rb < r1; rb += (int64_t)GEMV_WAVES * R) {
    const int64_t rn = rb + (int64_t)GEMV_WAVES * R;
    RawT nxt[R][NP];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const int64_t c = (int64_t)(pp * 64 + lane) * VEC;
        if (rn + rr < r1 && c < p.cols) nxt[rr][pp] = load_raw<T, VEC>(W + (rn + rr) * p.cols + c);
        else nxt[rr][pp] = RawT{};
      }
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
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) cur[rr][pp] = nxt[rr][pp];
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
    p.part_val[blockIdx.x] = v;
    p.part_idx[blockIdx.x] = ix;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(p.counter, 1u);
    s_last = (prev == (unsigned)(gridDim.x - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- pass 2 (last workgroup): best over all workgroups ----
  float v = -INFINITY;
  int ix = INT_MAX;
  for (int b = threadIdx.x; b < (int)gridDim.x; b += GEMV_THREADS) {
    const float bv = p.part_val[b];
    const int bi = p.part_idx[b];
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
    *p.counter = 0u;
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
  if (np <= 1) return head_one<T, VEC, 1, 8>(p, s);
  if (np <= 2) return head_one<T, VEC, 2, 4>(p, s);
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
