// Small kernels of the decode step for gfx950: residual add, add_rmsnorm, SiLU-gate, the RoPE table and
// RoPE, the in-place K/V append, the two-pass argmax, and state/fill helpers.
#include <float.h>
#include <limits.h>

#include "kernels.h"
#include "llmk.h"

namespace llmk {

constexpr int EW_THREADS = 256;

static unsigned grid_for(int64_t n, int per_block = EW_THREADS) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g > 65535LL * 16) g = 65535LL * 16;
  return (unsigned)(g < 1 ? 1 : g);
}

// ---- residual add ("LLM inference kernels", "Residual add") ---------------------------------------

__global__ void residual_add_kernel(const float* a, const float* b, float* out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = a[i] + b[i];
}

hipError_t residual_add_launch(const float* a, const float* b, float* out, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(residual_add_kernel, dim3(grid_for(n)), dim3(EW_THREADS), 0, s, a, b, out, n);
  return hipGetLastError();
}

// ---- add_rmsnorm ("decode-ops", "Usage"/"Method": residual += x, then RMSNorm with an fp32 square sum) ---

__global__ __launch_bounds__(EW_THREADS) void add_rmsnorm_kernel(float* residual, const float* x, const float* gain,
                                                                 int64_t n, float eps, float* h) {
  __shared__ float s_part[EW_THREADS / 64];
  const int64_t row = blockIdx.x;
  float* r = residual + row * n;
  const float* xr = x ? x + row * n : nullptr;
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += EW_THREADS) {
    float v = r[i];
    if (xr) {
      v = v + xr[i];
      r[i] = v;
    }
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  const float sc = 1.0f / sqrtf(tot / (float)n + eps);
  float* hr = h + row * n;
  for (int64_t i = threadIdx.x; i < n; i += EW_THREADS) hr[i] = r[i] * sc * gain[i];
}

hipError_t add_rmsnorm_launch(float* residual, const float* x, const float* gain, int64_t rows, int64_t n, float eps,
                              float* h, hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)rows), dim3(EW_THREADS), 0, s, residual, x, gain, n, eps, h);
  return hipGetLastError();
}

// ---- SiLU-gate ---------------------------------------------------------------------------------------

__global__ void silu_mul_kernel(const float* gate, const float* up, float* out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = silu_f(gate[i]) * up[i];
}

hipError_t silu_mul_launch(const float* gate, const float* up, float* out, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for(n)), dim3(EW_THREADS), 0, s, gate, up, out, n);
  return hipGetLastError();
}

// ---- RoPE table: angles and trig in fp64, stored fp32 ("decode-ops", "Method") -------------------------

__global__ void rope_table_kernel(float* table, int64_t max_pos, int64_t hd, double base) {
  const int64_t half = hd / 2, n = max_pos * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t pos = i / half, j = i % half;
    const double theta = (double)pos * pow(base, -(2.0 * (double)j) / (double)hd);
    table[i * 2 + 0] = (float)cos(theta);
    table[i * 2 + 1] = (float)sin(theta);
  }
}

hipError_t rope_table_launch(float* table, int64_t max_pos, int64_t hd, double base, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(max_pos * (hd / 2))), dim3(EW_THREADS), 0, s, table, max_pos, hd,
                     base);
  return hipGetLastError();
}

// ---- RoPE on q and k rows, row r at the device position pos[r] --------------------------------------------

__global__ void rope_kernel(float* q, float* k, int64_t rows, int64_t nq, int64_t nk, int64_t hd, const int32_t* pos,
                            int64_t max_pos, const float* table, int layout) {
  const int64_t half = hd / 2, per_row = (nq + nk) * half, n = rows * per_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, rem = i % per_row;
    const int64_t head = rem / half, j = rem % half;
    const int64_t p = pos[r];
    if (p < 0 || p >= max_pos) continue;   // no table row: the row stays as it is
    float* v = head < nq ? q + (r * nq + head) * hd : k + (r * nk + (head - nq)) * hd;
    const int64_t ia = layout == 0 ? j : 2 * j;
    const int64_t ib = layout == 0 ? j + half : 2 * j + 1;
    const float cs = table[(p * half + j) * 2 + 0];
    const float sn = table[(p * half + j) * 2 + 1];
    const float a = v[ia], b = v[ib];
    v[ia] = a * cs - b * sn;
    v[ib] = a * sn + b * cs;
  }
}

hipError_t rope_launch(float* q, float* k, int64_t rows, int64_t nq, int64_t nk, int64_t hd, const int32_t* pos,
                       int64_t max_pos, const float* table, int layout, hipStream_t s) {
  hipLaunchKernelGGL(rope_kernel, dim3(grid_for(rows * (nq + nk) * (hd / 2))), dim3(EW_THREADS), 0, s, q, k, rows, nq, nk,
                     hd, pos, max_pos, table, layout);
  return hipGetLastError();
}

// ---- prefill: RoPE on k and the K/V append of every row of a chunk, before any row attends ----------------

template <typename T>
__global__ void rope_append_rows_kernel(const float* qkv, int64_t qkv_stride, const BatchState* st, int32_t H,
                                        int32_t Hkv, int32_t hd, const float* table, int32_t layout, T* k, T* v,
                                        int64_t slot_elems, KvPaging pg) {
  const int r = blockIdx.x, kvh = blockIdx.y;
  const int64_t pos = st->pos[r];
  const float* src = qkv + (int64_t)r * qkv_stride;
  const float* ks = src + (int64_t)H * hd + (int64_t)kvh * hd;
  const float* vs = src + (int64_t)(H + Hkv) * hd + (int64_t)kvh * hd;
  const int64_t off = (pg.table ? kv_block_row(pg.table + (int64_t)st->slot[r] * pg.stride, pg.shift, pos) * Hkv * hd
                                : (int64_t)st->slot[r] * slot_elems + pos * Hkv * hd) + (int64_t)kvh * hd;
  const int half = hd / 2;
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const int ia = layout == 0 ? j : 2 * j;
    const int ib = layout == 0 ? j + half : 2 * j + 1;
    const float cs = table[(pos * half + j) * 2 + 0], sn = table[(pos * half + j) * 2 + 1];
    const float a = ks[ia], b = ks[ib];
    store_elem<T>(k + off, ia, a * cs - b * sn);
    store_elem<T>(k + off, ib, a * sn + b * cs);
  }
  for (int e = threadIdx.x; e < hd; e += blockDim.x) store_elem<T>(v + off, e, vs[e]);
}

// The int8 cache: one wave per (row, K/V head) rotates k into LDS, then quantizes k and v (s = max|x| / 127,
// codes rint(x / s) clamped to 127) and stores codes and scales.
__global__ __launch_bounds__(64) void rope_append_rows_q8_kernel(const float* qkv, int64_t qkv_stride,
                                                                 const BatchState* st, int32_t H, int32_t Hkv,
                                                                 int32_t hd, const float* table, int32_t layout,
                                                                 int8_t* k, int8_t* v, int64_t slot_elems,
                                                                 KvPaging pg, float* k_scale, float* v_scale) {
  __shared__ float s_x[2][256];
  const int r = blockIdx.x, kvh = blockIdx.y, lane = threadIdx.x;
  const int64_t pos = st->pos[r];
  const float* src = qkv + (int64_t)r * qkv_stride;
  const float* ks = src + (int64_t)H * hd + (int64_t)kvh * hd;
  const float* vs = src + (int64_t)(H + Hkv) * hd + (int64_t)kvh * hd;
  const int64_t crow = pg.table ? kv_block_row(pg.table + (int64_t)st->slot[r] * pg.stride, pg.shift, pos)
                                : (int64_t)st->slot[r] * (slot_elems / ((int64_t)Hkv * hd)) + pos;
  const int half = hd / 2;
  for (int j = lane; j < half; j += 64) {
    const int ia = layout == 0 ? j : 2 * j;
    const int ib = layout == 0 ? j + half : 2 * j + 1;
    const float cs = table[(pos * half + j) * 2 + 0], sn = table[(pos * half + j) * 2 + 1];
    const float a = ks[ia], b = ks[ib];
    s_x[0][ia] = a * cs - b * sn;
    s_x[0][ib] = a * sn + b * cs;
  }
  for (int e = lane; e < hd; e += 64) s_x[1][e] = vs[e];
  __syncthreads();
  for (int w = 0; w < 2; ++w) {
    float amax = 0.0f;
    for (int e = lane; e < hd; e += 64) amax = fmaxf(amax, fabsf(s_x[w][e]));
    const float sc = wave_max_dpp(amax) / 127.0f;
    int8_t* dst = (w == 0 ? k : v) + crow * Hkv * hd + (int64_t)kvh * hd;
    for (int e = lane; e < hd; e += 64)
      dst[e] = (int8_t)(sc > 0.0f ? fminf(fmaxf(rintf(s_x[w][e] / sc), -127.0f), 127.0f) : 0.0f);
    if (lane == 0) (w == 0 ? k_scale : v_scale)[crow * Hkv + kvh] = sc;
  }
}

hipError_t rope_append_rows_launch(const float* qkv, int64_t qkv_stride, const BatchState* st, int32_t rows,
                                   int32_t H, int32_t Hkv, int32_t hd, const float* rope_table, int32_t rope_layout,
                                   void* k, void* v, int32_t kv_dtype, int64_t slot_elems, const KvPaging& pg,
                                   float* k_scale, float* v_scale, hipStream_t s) {
  const dim3 grid((unsigned)rows, (unsigned)Hkv);
  if (kv_dtype == LLMK_Q8) {
    if (hd > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_append_rows_q8_kernel, grid, dim3(64), 0, s, qkv, qkv_stride, st, H, Hkv, hd, rope_table,
                       rope_layout, static_cast<int8_t*>(k), static_cast<int8_t*>(v), slot_elems, pg, k_scale, v_scale);
  } else if (kv_dtype == LLMK_BF16) {
    hipLaunchKernelGGL(rope_append_rows_kernel<bf16_t>, grid, dim3(64), 0, s, qkv, qkv_stride, st, H, Hkv, hd,
                       rope_table, rope_layout, static_cast<bf16_t*>(k), static_cast<bf16_t*>(v), slot_elems, pg);
  } else {
    hipLaunchKernelGGL(rope_append_rows_kernel<float>, grid, dim3(64), 0, s, qkv, qkv_stride, st, H, Hkv, hd,
                       rope_table, rope_layout, static_cast<float*>(k), static_cast<float*>(v), slot_elems, pg);
  }
  return hipGetLastError();
}

// ---- in-place K/V append: cache[offset + i] = round(src[i]) --------------------------------------------

__global__ void kv_append_kernel(void* cache, int is_bf16, int64_t offset, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (is_bf16) static_cast<bf16_t*>(cache)[offset + i] = f32_to_bf16(src[i]);
    else static_cast<float*>(cache)[offset + i] = src[i];
  }
}

hipError_t kv_append_launch(void* cache, int is_bf16, int64_t offset, const float* src, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid_for(n)), dim3(EW_THREADS), 0, s, cache, is_bf16, offset, src, n);
  return hipGetLastError();
}

// ---- greedy argmax: pass 1 per workgroup slice, pass 2 by the last workgroup of each row ---------------

__global__ __launch_bounds__(EW_THREADS) void argmax_kernel(const float* logits, int64_t n, int32_t* token, float* logit,
                                                            float* part_val, int32_t* part_idx, unsigned* counters) {
  __shared__ float s_v[EW_THREADS / 64];
  __shared__ int s_i[EW_THREADS / 64];
  __shared__ int s_last;
  const int64_t row = blockIdx.y;
  const int bpr = gridDim.x, b = blockIdx.x;
  const int64_t per = (n + bpr - 1) / bpr;
  const int64_t lo = b * per, hi = min(n, lo + per);
  const float* L = logits + row * n;
  float v = -INFINITY;
  int ix = INT_MAX;
  for (int64_t i = lo + threadIdx.x; i < hi; i += EW_THREADS) {
    const float x = L[i];
    if (argmax_better(x, (int)i, v, ix)) { v = x; ix = (int)i; }
  }
  wave_argmax(v, ix);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { s_v[wave] = v; s_i[wave] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = s_v[0];
    ix = s_i[0];
    for (int w = 1; w < EW_THREADS / 64; ++w)
      if (argmax_better(s_v[w], s_i[w], v, ix)) { v = s_v[w]; ix = s_i[w]; }
    st_dev(&part_val[row * bpr + b], v);
    st_dev(&part_idx[row * bpr + b], ix);
    stores_done();
    s_last = (take_ticket(&counters[row]) == (unsigned)(bpr - 1));
  }
  __syncthreads();
  if (!s_last) return;
  v = -INFINITY;
  ix = INT_MAX;
  for (int q = threadIdx.x; q < bpr; q += EW_THREADS) {
    const float bv = ld_dev(&part_val[row * bpr + q]);
    const int bi = ld_dev(&part_idx[row * bpr + q]);
    if (argmax_better(bv, bi, v, ix)) { v = bv; ix = bi; }
  }
  wave_argmax(v, ix);
  if (lane == 0) { s_v[wave] = v; s_i[wave] = ix; }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = s_v[0];
    ix = s_i[0];
    for (int w = 1; w < EW_THREADS / 64; ++w)
      if (argmax_better(s_v[w], s_i[w], v, ix)) { v = s_v[w]; ix = s_i[w]; }
    token[row] = ix;
    if (logit) logit[row] = v;
    reset_ticket(&counters[row]);
  }
}

hipError_t argmax_launch(const float* logits, int64_t rows, int64_t n, int32_t* token, float* logit, float* part_val,
                         int32_t* part_idx, unsigned* counters, int32_t blocks_per_row, hipStream_t s) {
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)blocks_per_row, (unsigned)rows), dim3(EW_THREADS), 0, s, logits, n,
                     token, logit, part_val, part_idx, counters);
  return hipGetLastError();
}

// ---- helpers ------------------------------------------------------------------------------------------

__global__ void fill_u32_kernel(unsigned* p, int64_t n, unsigned v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t fill_u32_launch(unsigned* p, int64_t n, unsigned v, hipStream_t s) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(EW_THREADS), 0, s, p, n, v);
  return hipGetLastError();
}

__global__ void set_state_kernel(DecodeState* st, int32_t token, int32_t pos) {
  if (threadIdx.x == 0) {
    st->token = token;
    st->pos = pos;
    st->step = 0;
    st->pad = 0;
  }
}

hipError_t set_state_launch(DecodeState* st, int32_t token, int32_t pos, hipStream_t s) {
  hipLaunchKernelGGL(set_state_kernel, dim3(1), dim3(64), 0, s, st, token, pos);
  return hipGetLastError();
}

}  // namespace llmk
