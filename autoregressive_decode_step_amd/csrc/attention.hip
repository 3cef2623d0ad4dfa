// Split-context grouped-query decode attention for gfx950.
//
// One query position; head h reads K/V head g = h / G (G = H / Hkv query heads share every K/V row,
// so each row is read once for all G of them). The context is cut into parts; a workgroup (4 waves)
// walks the consecutive sub-chunks of its part with an online softmax (running max and sum per head,
// output rescaled when the max grows), keeping the next sub-chunk's K and V rows in flight while it
// scores the current one. A row of hd elements is spread over hd/VEC lanes with 16-byte loads; the
// dot products reduce inside those lanes with xor shuffles. Each part writes (max, sum, unnormalised
// output) per head; the last workgroup of a K/V head merges the parts by log-sum-exp in part order:
// m* = max m_c, out = sum_c e^(m_c - m*) o_c / sum_c e^(m_c - m*) l_c.
// ("Inside the engine", "1. CausalLM": flash attention split across the context and reduced;
// "The forward pass end to end", "The code": the per-head softmax attention it computes.)
#include <float.h>

#include "kernels.h"

namespace llmk {

constexpr int ATTN_THREADS = 256;
constexpr int ATTN_WAVES = 4;
constexpr int ATTN_MAXC = 64;     // positions per sub-chunk, at most
constexpr int ATTN_MAXNI = 4;     // row loads per lane per sub-chunk, at most

template <typename T, int VEC, int G>
__global__ __launch_bounds__(ATTN_THREADS) void attn_kernel(const AttnParams p) {
  typedef typename Raw<T, VEC>::type RawT;
  __shared__ float s_p[G][ATTN_MAXC];
  __shared__ float s_alpha[G], s_m[G], s_l[G], s_inv[G];
  __shared__ float s_o[ATTN_WAVES][G][256];
  __shared__ float s_wm[ATTN_MAX_PARTS][G];
  __shared__ float s_wl[ATTN_MAX_PARTS][G];
  __shared__ int s_last;

  const int hd = p.hd, chunk = p.chunk;
  const int kvh = blockIdx.y, part = blockIdx.x;
  const int ctx = p.state ? p.state->pos + 1 : p.ctx;
  const int span = chunk * p.sub_per_wg;
  const int tb = part * span;
  if (tb >= ctx) return;
  const int te = min(tb + span, ctx);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int LPR = hd / VEC;               // lanes per row
  const int RPL = 64 / LPR;               // rows per wave load
  const int sub = lane % LPR, rsub = lane / LPR, e0 = sub * VEC;
  const int NI = (chunk + ATTN_WAVES * RPL - 1) / (ATTN_WAVES * RPL);
  const int64_t rstride = (int64_t)p.Hkv * hd;
  const T* Kb = static_cast<const T*>(p.k) + (int64_t)kvh * hd + e0;
  const T* Vb = static_cast<const T*>(p.v) + (int64_t)kvh * hd + e0;
  const float scale = 1.0f / sqrtf((float)hd);

  float qv[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < VEC; ++v) qv[g][v] = p.q[(int64_t)(kvh * G + g) * hd + e0 + v];

  float o[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[g][v] = 0.0f;
  if (threadIdx.x < G) { s_m[threadIdx.x] = -INFINITY; s_l[threadIdx.x] = 0.0f; }

  RawT kc[ATTN_MAXNI], vc[ATTN_MAXNI];
#pragma unroll
  for (int i = 0; i < ATTN_MAXNI; ++i) {
    const int t = tb + (i * ATTN_WAVES + wave) * RPL + rsub;
    if (i < NI && t < min(tb + chunk, te)) { kc[i] = load_raw<T, VEC>(Kb + t * rstride); vc[i] = load_raw<T, VEC>(Vb + t * rstride); }
    else { kc[i] = RawT{}; vc[i] = RawT{}; }
  }
  __syncthreads();

  for (int t0 = tb; t0 < te; t0 += chunk) {
    const int t1 = min(t0 + chunk, te);
    const int tn0 = t0 + chunk, tn1 = min(tn0 + chunk, te);
    RawT kn[ATTN_MAXNI], vn[ATTN_MAXNI];
#pragma unroll
    for (int i = 0; i < ATTN_MAXNI; ++i) {
      const int t = tn0 + (i * ATTN_WAVES + wave) * RPL + rsub;
      if (i < NI && t < tn1) { kn[i] = load_raw<T, VEC>(Kb + t * rstride); vn[i] = load_raw<T, VEC>(Vb + t * rstride); }
      else { kn[i] = RawT{}; vn[i] = RawT{}; }
    }
    // scores s_t = q . k_t / sqrt(hd)
#pragma unroll
    for (int i = 0; i < ATTN_MAXNI; ++i) {
      if (i < NI) {
        const int t = t0 + (i * ATTN_WAVES + wave) * RPL + rsub;
        float kf[VEC];
        unpack<T, VEC>(kc[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d = 0.0f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) d = fmaf(qv[g][v], kf[v], d);
          d = group_sum(d, LPR);
          if (sub == 0 && t < t1) s_p[g][t - t0] = d * scale;
        }
      }
    }
    __syncthreads();
    // online softmax update, one wave per head
    for (int g = wave; g < G; g += ATTN_WAVES) {
      const int n = t1 - t0;
      const float sv = lane < n ? s_p[g][lane] : -INFINITY;
      const float cm = wave_max(sv);
      const float m_old = s_m[g];
      const float m_new = fmaxf(m_old, cm);
      const float e = lane < n ? expf(sv - m_new) : 0.0f;
      const float es = wave_sum(e);
      if (lane < n) s_p[g][lane] = e;
      if (lane == 0) {
        const float alpha = expf(m_old - m_new);
        s_alpha[g] = alpha;
        s_l[g] = s_l[g] * alpha + es;
        s_m[g] = m_new;
      }
    }
    __syncthreads();
    // o = alpha * o + sum_t p_t v_t
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float a = s_alpha[g];
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[g][v] *= a;
    }
#pragma unroll
    for (int i = 0; i < ATTN_MAXNI; ++i) {
      const int t = t0 + (i * ATTN_WAVES + wave) * RPL + rsub;
      if (i < NI && t < t1) {
        float vf[VEC];
        unpack<T, VEC>(vc[i], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pr = s_p[g][t - t0];
#pragma unroll
          for (int v = 0; v < VEC; ++v) o[g][v] = fmaf(pr, vf[v], o[g][v]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ATTN_MAXNI; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
  }

  // reduce o over the row groups of each wave, then over the waves (fixed order)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      for (int off = 32; off >= LPR; off >>= 1) o[g][v] += __shfl_xor(o[g][v], off, 64);
  if (rsub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int v = 0; v < VEC; ++v) s_o[wave][g][e0 + v] = o[g][v];
  }
  __syncthreads();
  const int64_t pstride = hd + 2;
  float* P = p.part + ((int64_t)kvh * p.n_parts + part) * G * pstride;
  for (int idx = threadIdx.x; idx < G * hd; idx += ATTN_THREADS) {
    const int g = idx / hd, e = idx % hd;
    P[g * pstride + 2 + e] = ((s_o[0][g][e] + s_o[1][g][e]) + s_o[2][g][e]) + s_o[3][g][e];
  }
  if (threadIdx.x < G) {
    P[threadIdx.x * pstride + 0] = s_m[threadIdx.x];
    P[threadIdx.x * pstride + 1] = s_l[threadIdx.x];
  }

  // ---- last workgroup of this K/V head: log-sum-exp merge of the parts, in part order ----
  __threadfence();
  __syncthreads();
  const int np = (ctx + span - 1) / span;
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&p.counters[kvh], 1u);
    s_last = (prev == (unsigned)(np - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* PB = p.part + (int64_t)kvh * p.n_parts * G * pstride;
  for (int idx = threadIdx.x; idx < np * G; idx += ATTN_THREADS) {
    const int c = idx / G, g = idx % G;
    s_wm[c][g] = PB[(int64_t)(c * G + g) * pstride + 0];
    s_wl[c][g] = PB[(int64_t)(c * G + g) * pstride + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float ms = -INFINITY;
    for (int c = 0; c < np; ++c) ms = fmaxf(ms, s_wm[c][g]);
    float L = 0.0f;
    for (int c = 0; c < np; ++c) {
      const float w = expf(s_wm[c][g] - ms);
      s_wm[c][g] = w;
      L += s_wl[c][g] * w;
    }
    s_inv[g] = 1.0f / L;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * hd; idx += ATTN_THREADS) {
    const int g = idx / hd, e = idx % hd;
    float acc = 0.0f;
#pragma unroll 16
    for (int c = 0; c < np; ++c) acc = fmaf(s_wm[c][g], PB[(int64_t)(c * G + g) * pstride + 2 + e], acc);
    p.out[(int64_t)(kvh * G + g) * hd + e] = acc * s_inv[g];
  }
  if (threadIdx.x == 0) p.counters[kvh] = 0u;
}

void attn_plan(AttnParams& p, int64_t max_ctx) {
  const int vec = p.kv_is_bf16 ? 8 : 4;
  const int v = p.hd < vec ? 1 : vec;
  const int rpl = 64 / (p.hd / v);
  int chunk = ATTN_WAVES * rpl * ATTN_MAXNI;
  if (chunk > ATTN_MAXC) chunk = ATTN_MAXC;
  p.chunk = chunk;
  const int64_t n_sub = (max_ctx + chunk - 1) / chunk;
  const int64_t target = 32;
  int64_t spw = (n_sub + target - 1) / target;
  if (spw < 1) spw = 1;
  p.sub_per_wg = (int32_t)spw;
  p.n_parts = (int32_t)((n_sub + spw - 1) / spw);
}

template <typename T, int VEC, int G>
static hipError_t attn_one(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<T, VEC, G>), dim3((unsigned)p.n_parts, (unsigned)p.Hkv), dim3(ATTN_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename T, int VEC>
static hipError_t attn_g(const AttnParams& p, hipStream_t s) {
  switch (p.H / p.Hkv) {
    case 1: return attn_one<T, VEC, 1>(p, s);
    case 2: return attn_one<T, VEC, 2>(p, s);
    case 3: return attn_one<T, VEC, 3>(p, s);
    case 4: return attn_one<T, VEC, 4>(p, s);
    case 5: return attn_one<T, VEC, 5>(p, s);
    case 6: return attn_one<T, VEC, 6>(p, s);
    case 7: return attn_one<T, VEC, 7>(p, s);
    case 8: return attn_one<T, VEC, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t attn_launch(const AttnParams& p, hipStream_t s) {
  if (p.kv_is_bf16) return p.hd < 8 ? attn_g<bf16_t, 1>(p, s) : attn_g<bf16_t, 8>(p, s);
  return p.hd < 4 ? attn_g<float, 1>(p, s) : attn_g<float, 4>(p, s);
}

}  // namespace llmk
