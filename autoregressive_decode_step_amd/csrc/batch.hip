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

// The same with the row held in registers: d = 1024 NV, thread t holds elements 4 (t + 256 j) .. + 3 for j < NV,
// every load issued before the square sum, and x read from HBM once.
template <int NV>
__global__ __launch_bounds__(BN_THREADS) void bnorm_reg_kernel(float* x, const void* emb, int emb_is_bf16,
                                                               const BatchState* st, const float* gain, float eps,
                                                               bf16_t* hhi, bf16_t* hlo) {
  constexpr int64_t D = 1024 * NV;
  __shared__ float s_part[BN_THREADS / 64];
  const int b = blockIdx.x;
  float* xr = x + (int64_t)b * D;
  float4 v[NV];
  if (emb) {
    const int64_t tok = st->token[b];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t i = 4 * ((int64_t)threadIdx.x + BN_THREADS * j);
      if (emb_is_bf16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(emb) + tok * D + i);
        v[j] = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                           __uint_as_float(r.y & 0xFFFF0000u));
      } else {
        v[j] = *reinterpret_cast<const float4*>(static_cast<const float*>(emb) + tok * D + i);
      }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) *reinterpret_cast<float4*>(xr + 4 * ((int64_t)threadIdx.x + BN_THREADS * j)) = v[j];
  } else {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = *reinterpret_cast<const float4*>(xr + 4 * ((int64_t)threadIdx.x + BN_THREADS * j));
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    ss = fmaf(v[j].x, v[j].x, ss);
    ss = fmaf(v[j].y, v[j].y, ss);
    ss = fmaf(v[j].z, v[j].z, ss);
    ss = fmaf(v[j].w, v[j].w, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < BN_THREADS / 64; ++w) tot += s_part[w];
  const float scale = 1.0f / sqrtf(tot / (float)D + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t i = 4 * ((int64_t)threadIdx.x + BN_THREADS * j);
    const float4 g = *reinterpret_cast<const float4*>(gain + i);
    const float e[4] = {v[j].x * scale * g.x, v[j].y * scale * g.y, v[j].z * scale * g.z, v[j].w * scale * g.w};
    bf16_t h[4], l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) split_bf16(e[k], h[k], l[k]);
    *reinterpret_cast<uint2*>(hhi + (int64_t)b * D + i) =
        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    *reinterpret_cast<uint2*>(hlo + (int64_t)b * D + i) =
        make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
  }
}

hipError_t bnorm_launch(float* x, const void* emb, int emb_is_bf16, const BatchState* state, int32_t rows, int64_t d,
                        const float* gain, float eps, bf16_t* hhi, bf16_t* hlo, hipStream_t s) {
  const dim3 grid((unsigned)rows), block(BN_THREADS);
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  const bool vec_ok = al(x, 16) && al(gain, 16) && (!emb || al(emb, 16)) && al(hhi, 8) && al(hlo, 8);
  switch (vec_ok ? d : 0) {   // widths of 1,024..16,384 in steps of 1,024 that the register form takes
#define LLMK_BN_CASE(NV)                                                                                        \
  case 1024 * NV:                                                                                               \
    hipLaunchKernelGGL(bnorm_reg_kernel<NV>, grid, block, 0, s, x, emb, emb_is_bf16, state, gain, eps, hhi, hlo); \
    return hipGetLastError();
    LLMK_BN_CASE(1) LLMK_BN_CASE(2) LLMK_BN_CASE(3) LLMK_BN_CASE(4) LLMK_BN_CASE(5) LLMK_BN_CASE(6)
    LLMK_BN_CASE(8) LLMK_BN_CASE(12) LLMK_BN_CASE(16)
#undef LLMK_BN_CASE
  }
  hipLaunchKernelGGL(bnorm_kernel, grid, block, 0, s, x, emb, emb_is_bf16, state, d, gain, eps, hhi, hlo);
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
