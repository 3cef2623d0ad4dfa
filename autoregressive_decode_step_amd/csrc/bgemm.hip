// Batched decode projections on gfx950 matrix cores.
//
// With up to 64 sequences decoding together, every weight row is used by every row of the batch, so a
// projection becomes a skinny GEMM Y[b][n] = W[n] . X[b] ("Inside the engine", "5. The batched decode": one
// pass over the weights serves the whole batch). Weights stay bf16 and exact; the fp32 activations are
// carried as two bf16 parts, X = hi + lo, and each product is taken twice (W hi + W lo) into an fp32
// accumulator, so the result keeps about 16 significant bits of X instead of bf16's 8.
//
// v_mfma_f32_16x16x32_bf16: per wave, a 16 x 32 tile of W (lane l: row l % 16, eight consecutive k of
// group l / 16 -- one 16-byte load of a row) times a 32 x 16 tile of X (lane l: batch row l % 16, the same
// eight k) into a 16 x 16 fp32 tile (lane l: weight rows 4 (l / 16) .. + 3, batch row l % 16).
//
// A workgroup (4 waves) owns 64 weight rows (GATEUP: 32 gate rows and the same 32 up rows) and one slice
// of K; its waves take alternate 32-wide k steps over all 64 rows, so each X tile a wave loads serves four
// W tiles, and the four waves' partial sums are added in LDS in a fixed order. When K is split over
// several workgroups the slices' sums go to a partial buffer and the last workgroup of the row block
// (ticket) adds them in slice order and applies the epilogue. Each W byte is read once per step.
#include <limits.h>

#include "kernels.h"

namespace llmk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BG_THREADS = 256;
constexpr int BG_WAVES = 4;
constexpr int BG_STEP = 32;                   // k per matrix instruction
constexpr int BG_LDS = 68;                    // LDS row stride (floats) of the 64 weight rows of one batch row

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// weight row read by lane row i of tile t in row block rb (clamped to a valid row; `ok` false past N)
template <int MODE>
__device__ __forceinline__ const bf16_t* bg_row(const BgemmParams& p, int rb, int t, int i, bool& ok) {
  if (MODE == BG_GATEUP) {
    const int64_t o = (int64_t)rb * 32 + (t & 1) * 16 + i;
    ok = o < p.N;
    const int64_t oc = ok ? o : p.N - 1;
    return static_cast<const bf16_t*>(t < 2 ? p.w0 : p.w1) + oc * p.K;
  }
  const int64_t r = (int64_t)rb * 64 + t * 16 + i;
  ok = r < p.N;
  const int64_t rc = ok ? r : p.N - 1;
  if (MODE == BG_QKV) {
    if (rc < p.n0) return static_cast<const bf16_t*>(p.w0) + rc * p.K;
    if (rc < p.n0 + p.n1) return static_cast<const bf16_t*>(p.w1) + (rc - p.n0) * p.K;
    return static_cast<const bf16_t*>(p.w2) + (rc - p.n0 - p.n1) * p.K;
  }
  return static_cast<const bf16_t*>(p.w0) + rc * p.K;
}

template <int NB, int MODE>
__global__ __launch_bounds__(BG_THREADS) void bgemm_kernel(const BgemmParams p) {
  __shared__ float red[BG_WAVES][NB * 16][BG_LDS];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x % p.n_rblk, ks = blockIdx.x / p.n_rblk;
  const int64_t k0 = (int64_t)ks * p.kslice;
  const int64_t k1 = min(p.K, k0 + p.kslice);
  const int nsteps = (int)((k1 - k0 + BG_STEP - 1) / BG_STEP);
  const int li = lane & 15, kg = lane >> 4;
  const int64_t kl = k0 + 8 * kg;              // this lane's first k within a step

  const bf16_t* arow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bool ok;
    arow[t] = bg_row<MODE>(p, rb, t, li, ok) + kl;
  }
  const bf16_t* xh[NB];
  const bf16_t* xl[NB];
  bool bok[NB];
#pragma unroll
  for (int bt = 0; bt < NB; ++bt) {
    const int b = bt * 16 + li;
    bok[bt] = b < p.B;
    const int64_t off = (int64_t)(bok[bt] ? b : 0) * p.K + kl;
    xh[bt] = p.xhi + off;
    xl[bt] = p.xlo + off;
  }

  f32x4_t acc[4][NB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) acc[t][bt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // wave w takes steps w, w + 4, w + 8, ... (its j-th step is w + 4 j). W tiles are requested 4 steps
  // ahead (ring a[4]), X tiles one step ahead (b[2]); the register file holds one wave per SIMD, so the
  // loads in flight come from depth, not from occupancy
  constexpr int DA = 4;
  uint4 a[DA][4], bh[2][NB], bl[2][NB];
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const int nj = nsteps > wave ? (nsteps - wave + BG_WAVES - 1) / BG_WAVES : 0;
  // k past the slice end (the last step of a K that is not a multiple of 32) contributes zero
#define LLMK_BG_LOAD_A(BUF, J)                                                                 \
  {                                                                                            \
    const int64_t off_ = (int64_t)(wave + BG_WAVES * (J)) * BG_STEP;                           \
    const bool kin_ = kl + off_ < k1;                                                          \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                              \
      a[BUF][t] = kin_ ? *reinterpret_cast<const uint4*>(arow[t] + off_) : zero;               \
  }
#define LLMK_BG_LOAD_B(BUF, J)                                                                 \
  {                                                                                            \
    const int64_t off_ = (int64_t)(wave + BG_WAVES * (J)) * BG_STEP;                           \
    const bool kin_ = kl + off_ < k1;                                                          \
    _Pragma("unroll") for (int bt = 0; bt < NB; ++bt) {                                        \
      bh[BUF][bt] = (kin_ && bok[bt]) ? *reinterpret_cast<const uint4*>(xh[bt] + off_) : zero; \
      bl[BUF][bt] = (kin_ && bok[bt]) ? *reinterpret_cast<const uint4*>(xl[bt] + off_) : zero; \
    }                                                                                          \
  }
#define LLMK_BG_STEP(I)                                                                        \
  {                                                                                            \
    const int j_ = j0 + (I);                                                                   \
    if (j_ >= nj) break;                                                                       \
    if (j_ + 1 < nj) LLMK_BG_LOAD_B(((I) + 1) & 1, j_ + 1)                                     \
    _Pragma("unroll") for (int t = 0; t < 4; ++t)                                              \
      _Pragma("unroll") for (int bt = 0; bt < NB; ++bt) {                                      \
        acc[t][bt] = mfma_bf16(a[I][t], bh[(I) & 1][bt], acc[t][bt]);                          \
        acc[t][bt] = mfma_bf16(a[I][t], bl[(I) & 1][bt], acc[t][bt]);                          \
      }                                                                                        \
    if (j_ + DA < nj) LLMK_BG_LOAD_A(I, j_ + DA)                                               \
  }

#pragma unroll
  for (int i = 0; i < DA; ++i)
    if (i < nj) LLMK_BG_LOAD_A(i, i)
  if (nj > 0) LLMK_BG_LOAD_B(0, 0)
  for (int j0 = 0; j0 < nj; j0 += DA) {
    LLMK_BG_STEP(0)
    LLMK_BG_STEP(1)
    LLMK_BG_STEP(2)
    LLMK_BG_STEP(3)
  }
#undef LLMK_BG_LOAD_A
#undef LLMK_BG_LOAD_B
#undef LLMK_BG_STEP

  // ---- the four waves' sums, per (batch row, local weight row), in LDS ----
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      float* dst = &red[wave][bt * 16 + li][t * 16 + 4 * kg];
      *reinterpret_cast<float4*>(dst) = make_float4(acc[t][bt][0], acc[t][bt][1], acc[t][bt][2], acc[t][bt][3]);
    }
  __syncthreads();
  constexpr int NV = NB * 16 * 64;
  const int64_t RT = (int64_t)p.n_rblk * 64;   // partial row length
  if (p.ksplit > 1) {
    for (int i = threadIdx.x; i < NV; i += BG_THREADS) {
      const int b = i >> 6, lr = i & 63;
      if (b < p.B) {
        const float v = red[0][b][lr] + red[1][b][lr] + red[2][b][lr] + red[3][b][lr];
        st_dev(&p.partial[((int64_t)ks * 64 + b) * RT + (int64_t)rb * 64 + lr], v);
      }
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (take_ticket(&p.counters[rb]) == (unsigned)(p.ksplit - 1));
    __syncthreads();
    if (!s_last) return;
    for (int i = threadIdx.x; i < NV; i += BG_THREADS) {
      const int b = i >> 6, lr = i & 63;
      if (b < p.B) {
        float v = 0.0f;
        for (int k = 0; k < p.ksplit; ++k) v += ld_dev(&p.partial[((int64_t)k * 64 + b) * RT + (int64_t)rb * 64 + lr]);
        red[0][b][lr] = v;
      }
    }
    if (threadIdx.x == 0) reset_ticket(&p.counters[rb]);
  } else {
    for (int i = threadIdx.x; i < NV; i += BG_THREADS) {
      const int b = i >> 6, lr = i & 63;
      red[0][b][lr] = red[0][b][lr] + red[1][b][lr] + red[2][b][lr] + red[3][b][lr];
    }
  }
  __syncthreads();

  // ---- epilogue: red[0][b][lr] holds y of batch row b, local weight row lr ----
  if (MODE == BG_GATEUP) {
    for (int i = threadIdx.x; i < NB * 16 * 32; i += BG_THREADS) {
      const int b = i >> 5, o = i & 31;
      const int64_t n = (int64_t)rb * 32 + o;
      if (b < p.B && n < p.N) {
        const float u = silu_f(red[0][b][o]) * red[0][b][o + 32];
        bf16_t hi, lo;
        split_bf16(u, hi, lo);
        p.uhi[(int64_t)b * p.N + n] = hi;
        p.ulo[(int64_t)b * p.N + n] = lo;
      }
    }
    return;
  }
  if (MODE == BG_HEAD) {
    // logits, then per batch row this block's best (wave w takes rows w, w + 4, ...; lanes the 64 weight rows)
    for (int b = wave; b < NB * 16; b += BG_WAVES) {
      const int64_t n = (int64_t)rb * 64 + lane;
      float v = -INFINITY;
      int ix = INT_MAX;
      if (b < p.B && n < p.N) {
        v = red[0][b][lane];
        ix = (int)n;
        if (p.y) p.y[(int64_t)b * p.N + n] = v;
      }
      wave_argmax(v, ix);
      if (b < p.B && lane == 0) {
        st_dev(&p.part_val[(int64_t)b * p.n_rblk + rb], v);
        st_dev(&p.part_idx[(int64_t)b * p.n_rblk + rb], ix);
      }
    }
    stores_done();
    __syncthreads();
    unsigned* cnt = p.counters + p.n_rblk;
    if (threadIdx.x == 0) s_last = (take_ticket(cnt) == (unsigned)(p.n_rblk - 1));
    __syncthreads();
    if (!s_last) return;
    const int step = p.state->step;
    for (int b = wave; b < p.B; b += BG_WAVES) {
      float v = -INFINITY;
      int ix = INT_MAX;
      for (int j = lane; j < p.n_rblk; j += 64) {
        const float bv = ld_dev(&p.part_val[(int64_t)b * p.n_rblk + j]);
        const int bi = ld_dev(&p.part_idx[(int64_t)b * p.n_rblk + j]);
        if (argmax_better(bv, bi, v, ix)) { v = bv; ix = bi; }
      }
      wave_argmax(v, ix);
      if (lane == 0) {
        p.token_out[(int64_t)step * p.B + b] = ix;
        p.state->token[b] = ix;
        p.state->pos[b] = p.state->pos[b] + 1;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      p.state->step = step + 1;
      reset_ticket(cnt);
    }
    return;
  }
  for (int i = threadIdx.x; i < NV; i += BG_THREADS) {
    const int b = i >> 6, lr = i & 63;
    const int64_t n = (int64_t)rb * 64 + lr;
    if (b >= p.B || n >= p.N) continue;
    const float v = red[0][b][lr];
    if (MODE == BG_RESID) {
      const float xo = p.x[(int64_t)b * p.N + n] + v;
      p.x[(int64_t)b * p.N + n] = xo;
      if (p.hidden) p.hidden[(int64_t)b * p.hidden_stride + n] = xo;
    } else {
      p.y[(int64_t)b * p.N + n] = v;
    }
  }
}

void bgemm_plan(BgemmParams& p, int mode, int target_blocks) {
  p.n_rblk = (int32_t)(mode == BG_GATEUP ? (p.N + 31) / 32 : (p.N + 63) / 64);
  int64_t ks = target_blocks / p.n_rblk;
  if (ks < 1 || mode == BG_HEAD) ks = 1;
  const int64_t unit = BG_STEP * BG_WAVES;     // every wave gets whole steps
  int64_t slice = (p.K + ks - 1) / ks;
  slice = (slice + unit - 1) / unit * unit;
  if (slice < 4 * unit) slice = 4 * unit;      // at least 4 steps per wave
  p.kslice = slice;
  p.ksplit = (int32_t)((p.K + slice - 1) / slice);
}

int64_t bgemm_partial_floats(const BgemmParams& p) {
  return p.ksplit > 1 ? (int64_t)p.ksplit * 64 * p.n_rblk * 64 : 0;
}

template <int NB, int MODE>
static hipError_t bg_one(const BgemmParams& p, hipStream_t s) {
  hipLaunchKernelGGL((bgemm_kernel<NB, MODE>), dim3((unsigned)(p.n_rblk * p.ksplit)), dim3(BG_THREADS), 0, s, p);
  return hipGetLastError();
}

template <int MODE>
static hipError_t bg_nb(const BgemmParams& p, hipStream_t s) {
  switch ((p.B + 15) / 16) {
    case 1: return bg_one<1, MODE>(p, s);
    case 2: return bg_one<2, MODE>(p, s);
    case 3: return bg_one<3, MODE>(p, s);
    case 4: return bg_one<4, MODE>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t bgemm_launch(const BgemmParams& p, int mode, hipStream_t s) {
  if (p.B < 1 || p.B > LLMK_MAX_BATCH_ROWS || p.K % 8 != 0) return hipErrorInvalidValue;
  switch (mode) {
    case BG_PLAIN: return bg_nb<BG_PLAIN>(p, s);
    case BG_QKV: return bg_nb<BG_QKV>(p, s);
    case BG_RESID: return bg_nb<BG_RESID>(p, s);
    case BG_GATEUP: return bg_nb<BG_GATEUP>(p, s);
    case BG_HEAD: return bg_nb<BG_HEAD>(p, s);
  }
  return hipErrorInvalidValue;
}

// ---- per-row RMSNorm into hi/lo parts (and the embedding gather of the first layer) ----

constexpr int BN_THREADS = 256;

__global__ __launch_bounds__(BN_THREADS) void bnorm_kernel(float* x, const void* emb, int emb_is_bf16,
                                                           const BatchState* st, int64_t d, const float* gain,
                                                           float eps, bf16_t* hhi, bf16_t* hlo) {
  __shared__ float s_part[BN_THREADS / 64];
  const int b = blockIdx.x;
  float* xr = x + (int64_t)b * d;
  if (emb) {
    const int64_t tok = st->token[b];
    for (int64_t i = threadIdx.x; i < d; i += BN_THREADS)
      xr[i] = emb_is_bf16 ? bf16_to_f32(static_cast<const bf16_t*>(emb)[tok * d + i])
                          : static_cast<const float*>(emb)[tok * d + i];
  }
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < d; i += BN_THREADS) ss = fmaf(xr[i], xr[i], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < BN_THREADS / 64; ++w) tot += s_part[w];
  const float scale = 1.0f / sqrtf(tot / (float)d + eps);
  for (int64_t i = threadIdx.x; i < d; i += BN_THREADS) {
    bf16_t hi, lo;
    split_bf16(xr[i] * scale * gain[i], hi, lo);
    hhi[(int64_t)b * d + i] = hi;
    hlo[(int64_t)b * d + i] = lo;
  }
}

hipError_t bnorm_launch(float* x, const void* emb, int emb_is_bf16, const BatchState* state, int32_t rows, int64_t d,
                        const float* gain, float eps, bf16_t* hhi, bf16_t* hlo, hipStream_t s) {
  hipLaunchKernelGGL(bnorm_kernel, dim3((unsigned)rows), dim3(BN_THREADS), 0, s, x, emb, emb_is_bf16, state, d, gain,
                     eps, hhi, hlo);
  return hipGetLastError();
}

__global__ void set_batch_state_kernel(BatchState* st, const BatchInit init) {
  const int i = threadIdx.x;
  if (i < LLMK_MAX_BATCH_ROWS) {
    st->token[i] = init.token[i];
    st->pos[i] = init.pos[i];
    st->slot[i] = init.slot[i];
  }
  if (i == 0) {
    st->rows = init.rows;
    st->step = 0;
    st->pad[0] = st->pad[1] = 0;
  }
}

__global__ void batch_advance_kernel(BatchState* st, const int32_t* tok, int32_t* token_out, int32_t rows) {
  const int step = st->step;
  for (int b = threadIdx.x; b < rows; b += blockDim.x) {
    const int32_t t = tok[b];
    token_out[(int64_t)step * rows + b] = t;
    st->token[b] = t;
    st->pos[b] = st->pos[b] + 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) st->step = step + 1;
}

hipError_t batch_advance_launch(BatchState* st, const int32_t* tok, int32_t* token_out, int32_t rows, hipStream_t s) {
  hipLaunchKernelGGL(batch_advance_kernel, dim3(1), dim3(64), 0, s, st, tok, token_out, rows);
  return hipGetLastError();
}

hipError_t set_batch_state_launch(BatchState* st, const BatchInit& init, hipStream_t s) {
  hipLaunchKernelGGL(set_batch_state_kernel, dim3(1), dim3(LLMK_MAX_BATCH_ROWS), 0, s, st, init);
  return hipGetLastError();
}

}  // namespace llmk
