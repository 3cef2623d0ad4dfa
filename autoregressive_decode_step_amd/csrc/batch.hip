// Row helpers of the batched decode step and of prefill chunks on gfx950: the per-row RMSNorm into the bf16
// hi + lo parts the matrix-core projections take (with the first layer's embedding gather), the device-side
// row state (token, position, slot per row), and its advance after the head's argmax.
//
// The projections themselves run on the tiled matrix-core GEMM of pgemm.hip: with 64 decode rows it re-reads
// the activations from L2 less than a skinny one-pass-over-the-weights kernel does ("Inside the engine",
// "5. The batched decode": one pass over the weights serves the whole batch; here one pass per 128 rows).
#include "kernels.h"

namespace llmk {

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
