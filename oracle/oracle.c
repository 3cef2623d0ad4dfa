/*
 * THE ORACLE -- test infrastructure only.
 *
 * A plain, slow, obviously correct CPU implementation of one greedy decode step of a
 * Llama/Qwen-style grouped-query decoder, written from the pages' definitions:
 *   [llmk]  "LLM inference kernels" (docs.algenta.ai)
 *   [dops]  "decode-ops" (Hugging Face kernels page)
 *   [xpu]   "Inside the engine" (cajeta.dev)
 *   [fwd]   "The forward pass end to end: a Llama-style engine in 100 lines" (inferenceacademy.com)
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this code. It shares no source, header or helper with the GPU library and the GPU
 * library never calls it.
 *
 * Arithmetic: every value is computed in fp64 from the exact stored inputs (fp32, bf16
 * and fp64 inputs all convert to double exactly). Values are rounded only where the
 * method stores them: logits, hidden states and primitive outputs to fp32, and K/V to
 * the cache dtype (via fp32; bf16 by round-to-nearest-even). Loops run in the order the
 * definitions state; OpenMP splits only independent outputs (gemv columns, matvec rows,
 * attention heads), so results do not depend on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_Q8 = 3 };
enum { ORC_HALF_SPLIT = 0, ORC_INTERLEAVED = 1 };

/* ---- storage types ------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is a 16-bit shift, exact. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even; a NaN stays a (quiet) NaN. */
static uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static double load(const void* base, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)base)[i]);
  return ((const double*)base)[i];
}

/* Store v rounded to the storage dtype: fp32 by one rounding, bf16 via fp32 then RNE. */
static void store(void* base, int dtype, int64_t i, double v) {
  if (dtype == ORC_F32) ((float*)base)[i] = (float)v;
  else if (dtype == ORC_BF16) ((uint16_t*)base)[i] = float_to_bf16((float)v);
  else ((double*)base)[i] = v;
}

double orc_bf16_to_double(uint16_t b) { return bf16_to_double(b); }

/* int8 K/V rows. The pages name int8 K/V caches ("decode-ops", its opening paragraph: the int8-KV CPU
 * attention; "Inside the engine", "1. CausalLM": int8 copies) without fixing a format, so this is the
 * library's own, defined here: one row of n values (a position's K or V for one K/V head) is kept as n int8
 * codes and one fp32 scale. Each value is first rounded to fp32 (as for every cache dtype); the scale is
 * s = max|x| / 127 (one fp32 division); a code is q = rint(x / s) (one fp32 division, ties to even),
 * clamped to [-127, 127]; a row of zeros has s = 0 and codes 0. The value the row stands for is q * s,
 * exact in fp64, so |x - q s| <= s / 2 for every element (plus the fp32 rounding of x and of x / s). */
void orc_q8_row(const double* x, int64_t n, int8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    const float a = fabsf((float)x[i]);
    if (a > amax) amax = a;
  }
  const float s = amax / 127.0f;
  for (int64_t i = 0; i < n; ++i) {
    float r = s > 0.0f ? rintf((float)x[i] / s) : 0.0f;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
  *s_out = s;
}

/* A layer's int8 cache buffer: codes [max_seq][n_kv][hd], then scales fp32 [max_seq][n_kv]. */
static float q8_scale(const void* buf, int64_t codes_bytes, int64_t row) {
  float s;
  memcpy(&s, (const char*)buf + codes_bytes + 4 * row, 4);
  return s;
}
static void q8_store_row(void* buf, int64_t codes_bytes, int64_t row, int64_t hd, const double* x) {
  float s;
  orc_q8_row(x, hd, (int8_t*)buf + row * hd, &s);
  memcpy((char*)buf + codes_bytes + 4 * row, &s, 4);
}
/* Rows 0..n-1 of a layer's int8 cache as the values they stand for (q * s), [n][n_kv][hd] fp64. */
static void q8_dequantize(const void* buf, int64_t codes_bytes, int64_t n_rows, int64_t hd, double* out) {
  for (int64_t r = 0; r < n_rows; ++r) {
    const double s = (double)q8_scale(buf, codes_bytes, r);
    for (int64_t i = 0; i < hd; ++i) out[r * hd + i] = (double)((const int8_t*)buf)[r * hd + i] * s;
  }
}

/* Softmax of each row of s [rows][cols] over its first last[r] + 1 entries, in place: the maximum subtracted,
 * exp, divided by the sum; entries past last[r] become 0 (positions a query row does not see). Rows are
 * independent, so OpenMP splits them. */
void orc_softmax_rows(double* s, int64_t rows, int64_t cols, const int64_t* last) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double* row = s + r * cols;
    const int64_t n = last[r] + 1 < cols ? last[r] + 1 : cols;
    double m = row[0];
    for (int64_t t = 1; t < n; ++t) if (row[t] > m) m = row[t];
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) { row[t] = exp(row[t] - m); sum += row[t]; }
    for (int64_t t = 0; t < n; ++t) row[t] /= sum;
    for (int64_t t = n; t < cols; ++t) row[t] = 0.0;
  }
}

double orc_silu(double z);

/* g[i] = silu(g[i]) * u[i] in place (fp64), elements split over OpenMP threads. */
void orc_silu_mul_inplace(double* g, const double* u, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) g[i] = orc_silu(g[i]) * u[i];
}

/* Widen n stored values (fp32 or bf16) to fp64, exactly; elements are independent, so OpenMP splits them. */
void orc_widen(const void* src, int dtype, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = load(src, dtype, i);
}
uint16_t orc_float_to_bf16(float f) { return float_to_bf16(f); }

/* ---- the primitives ------------------------------------------------------------------ */

/* y = A^T x with A m x n row-major: y[j] = sum over i = 0..m-1 of A[i][j] x[i].
 * [llmk] "A parallel path for one frozen kernel's known-slow shape": the output columns are split
 * into contiguous bands, and inside its band each worker walks the rows of A in order (i outer,
 * j inner), so every y[j] is summed over i in ascending order whatever the thread count. */
void orc_gemv_t(const void* a, int a_dtype, const double* x, int64_t m, int64_t n, double* y) {
#pragma omp parallel
  {
    int64_t nt = omp_get_num_threads(), t = omp_get_thread_num();
    int64_t j0 = n * t / nt, j1 = n * (t + 1) / nt;
    for (int64_t j = j0; j < j1; ++j) y[j] = 0.0;
    for (int64_t i = 0; i < m; ++i) {
      const double xi = x[i];
      if (a_dtype == ORC_BF16) {
        const uint16_t* row = (const uint16_t*)a + i * n;
        for (int64_t j = j0; j < j1; ++j) y[j] += bf16_to_double(row[j]) * xi;
      } else if (a_dtype == ORC_F32) {
        const float* row = (const float*)a + i * n;
        for (int64_t j = j0; j < j1; ++j) y[j] += (double)row[j] * xi;
      } else {
        const double* row = (const double*)a + i * n;
        for (int64_t j = j0; j < j1; ++j) y[j] += row[j] * xi;
      }
    }
  }
}

/* y = W x with W rows x cols row-major: y[r] = sum over c of W[r][c] x[c]
 * ([fwd] "The code": matvec, one dot product per row; the untransposed output head). */
void orc_matvec(const void* w, int w_dtype, const double* x, int64_t rows, int64_t cols, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += load(w, w_dtype, r * cols + c) * x[c];
    y[r] = s;
  }
}

/* out = x * (mean(x^2) + eps)^(-1/2) * g  ([fwd] "The code": rmsnorm; eps inside the mean). */
void orc_rmsnorm(const double* x, const float* g, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double s = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * s * (double)g[i];
}

/* silu(z) = z / (1 + e^-z)  ([fwd] "The code"; [dops] "Usage": silu_mul). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Rotate every head of v (n_heads x hd) by position pos. Pair j (0 <= j < hd/2) is turned by
 * theta = pos * base^(-2j/hd), angles in fp64 ([dops] "Method"). Half-split pairs are (j, j + hd/2)
 * (GPT-NeoX / Qwen3, [llmk] "Two gaps, not three"); interleaved pairs are (2j, 2j+1) ([fwd] "The
 * code": rope, whose exponent -i/hd with i = 2j is the same angle). (a, b) -> (a cos - b sin,
 * a sin + b cos). */
void orc_rope(double* v, int64_t n_heads, int64_t hd, int64_t pos, double base, int layout) {
  const int64_t half = hd / 2;
  for (int64_t h = 0; h < n_heads; ++h) {
    double* vh = v + h * hd;
    for (int64_t j = 0; j < half; ++j) {
      const double theta = (double)pos * pow(base, -(2.0 * (double)j) / (double)hd);
      const double c = cos(theta), s = sin(theta);
      const int64_t ia = layout == ORC_INTERLEAVED ? 2 * j : j;
      const int64_t ib = layout == ORC_INTERLEAVED ? 2 * j + 1 : j + half;
      const double a = vh[ia], b = vh[ib];
      vh[ia] = a * c - b * s;
      vh[ib] = a * s + b * c;
    }
  }
}

/* Grouped-query attention of one query position over ctx cached positions.
 * For head h, K/V head g = h / (n_head / n_kv); s_t = (q_h . K[t][g]) / sqrt(hd) for t < ctx;
 * w = softmax(s) with the maximum subtracted; out_h[i] = sum_t w_t V[t][g][i]
 * ([fwd] "The code": forward_token's per-head loop and softmax). K, V: [ctx][n_kv][hd] of kv_dtype. */
void orc_attend(const double* q, const void* k, const void* v, int kv_dtype, int64_t ctx, int64_t n_head,
                int64_t n_kv, int64_t hd, double* out) {
  const int64_t group = n_head / n_kv;
#pragma omp parallel for schedule(static)
  for (int64_t h = 0; h < n_head; ++h) {
    const int64_t g = h / group;
    double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
    for (int64_t t = 0; t < ctx; ++t) {
      double dot = 0.0;
      for (int64_t i = 0; i < hd; ++i) dot += q[h * hd + i] * load(k, kv_dtype, (t * n_kv + g) * hd + i);
      s[t] = dot / sqrt((double)hd);
    }
    double m = s[0];
    for (int64_t t = 1; t < ctx; ++t) if (s[t] > m) m = s[t];
    double sum = 0.0;
    for (int64_t t = 0; t < ctx; ++t) { s[t] = exp(s[t] - m); sum += s[t]; }
    for (int64_t t = 0; t < ctx; ++t) s[t] /= sum;
    for (int64_t i = 0; i < hd; ++i) {
      double o = 0.0;
      for (int64_t t = 0; t < ctx; ++t) o += s[t] * load(v, kv_dtype, (t * n_kv + g) * hd + i);
      out[h * hd + i] = o;
    }
    free(s);
  }
}

/* Greedy argmax of n fp32 logits in two passes ([llmk] "KV-cache growth and greedy argmax"):
 * pass 1 finds the row's maximum, pass 2 returns the first id equal to it, so ties go to the
 * lowest id. +0.0 == -0.0. NaN counts as larger than every number and the first NaN wins (the
 * numpy/torch argmax convention the pages point to). Writes the winning value to *best. */
int64_t orc_argmax_f32(const float* v, int64_t n, float* best) {
  int any_nan = 0;
  float m = v[0];
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(v[i])) { any_nan = 1; break; }
    if (v[i] > m) m = v[i];
  }
  for (int64_t i = 0; i < n; ++i) {
    if (any_nan ? isnan(v[i]) : v[i] == m) {
      if (best) *best = v[i];
      return i;
    }
  }
  return -1; /* unreachable for n >= 1 */
}

/* ---- fp32-in / fp32-out forms of the primitives, for element-by-element parity --------- */

void orc_gemv_t_f32(const void* a, int a_dtype, const float* x, int64_t m, int64_t n, float* y) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)m);
  double* yd = (double*)malloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < m; ++i) xd[i] = (double)x[i];
  orc_gemv_t(a, a_dtype, xd, m, n, yd);
  for (int64_t j = 0; j < n; ++j) y[j] = (float)yd[j];
  free(xd); free(yd);
}

void orc_matvec_f32(const void* w, int w_dtype, const float* x, int64_t rows, int64_t cols, float* y) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)cols);
  double* yd = (double*)malloc(sizeof(double) * (size_t)rows);
  for (int64_t c = 0; c < cols; ++c) xd[c] = (double)x[c];
  orc_matvec(w, w_dtype, xd, rows, cols, yd);
  for (int64_t r = 0; r < rows; ++r) y[r] = (float)yd[r];
  free(xd); free(yd);
}

/* out[i] = a[i] + b[i] ([llmk] "Residual add"). */
void orc_residual_add_f32(const float* a, const float* b, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)((double)a[i] + (double)b[i]);
}

/* Per row: if x != NULL, residual += x (stored fp32); h = rmsnorm(residual) * gain
 * ([dops] "Usage": add_rmsnorm -- residual += x, then norm). */
void orc_add_rmsnorm_f32(float* residual, const float* x, const float* gain, int64_t rows, int64_t n, double eps,
                         float* h) {
  double* r = (double*)malloc(sizeof(double) * (size_t)n);
  double* o = (double*)malloc(sizeof(double) * (size_t)n);
  for (int64_t row = 0; row < rows; ++row) {
    float* rr = residual + row * n;
    if (x) for (int64_t i = 0; i < n; ++i) rr[i] = (float)((double)rr[i] + (double)x[row * n + i]);
    for (int64_t i = 0; i < n; ++i) r[i] = (double)rr[i];
    orc_rmsnorm(r, gain, n, eps, o);
    for (int64_t i = 0; i < n; ++i) h[row * n + i] = (float)o[i];
  }
  free(r); free(o);
}

/* out[i] = silu(gate[i]) * up[i]. */
void orc_silu_mul_f32(const float* gate, const float* up, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(orc_silu((double)gate[i]) * (double)up[i]);
}

/* In-place RoPE of q [rows][n_q][hd] and k [rows][n_k][hd], row r at position pos0 + r. */
void orc_rope_f32(float* q, float* k, int64_t rows, int64_t n_q, int64_t n_k, int64_t hd, int64_t pos0, double base,
                  int layout) {
  const int64_t wq = n_q * hd, wk = n_k * hd;
  double* buf = (double*)malloc(sizeof(double) * (size_t)(wq > wk ? wq : wk));
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < wq; ++i) buf[i] = (double)q[r * wq + i];
    orc_rope(buf, n_q, hd, pos0 + r, base, layout);
    for (int64_t i = 0; i < wq; ++i) q[r * wq + i] = (float)buf[i];
    if (k) {
      for (int64_t i = 0; i < wk; ++i) buf[i] = (double)k[r * wk + i];
      orc_rope(buf, n_k, hd, pos0 + r, base, layout);
      for (int64_t i = 0; i < wk; ++i) k[r * wk + i] = (float)buf[i];
    }
  }
  free(buf);
}

/* The cos/sin table a GPU RoPE reads: table[(p*(hd/2) + j)*2 + {0,1}] = {cos, sin}(p base^(-2j/hd)). */
void orc_rope_table_f32(int64_t max_pos, int64_t hd, double base, float* table) {
  const int64_t half = hd / 2;
  for (int64_t p = 0; p < max_pos; ++p)
    for (int64_t j = 0; j < half; ++j) {
      const double theta = (double)p * pow(base, -(2.0 * (double)j) / (double)hd);
      table[(p * half + j) * 2 + 0] = (float)cos(theta);
      table[(p * half + j) * 2 + 1] = (float)sin(theta);
    }
}

void orc_attend_f32(const float* q, const void* k, const void* v, int kv_dtype, int64_t ctx, int64_t n_head,
                    int64_t n_kv, int64_t hd, float* out) {
  double* qd = (double*)malloc(sizeof(double) * (size_t)(n_head * hd));
  double* od = (double*)malloc(sizeof(double) * (size_t)(n_head * hd));
  for (int64_t i = 0; i < n_head * hd; ++i) qd[i] = (double)q[i];
  orc_attend(qd, k, v, kv_dtype, ctx, n_head, n_kv, hd, od);
  for (int64_t i = 0; i < n_head * hd; ++i) out[i] = (float)od[i];
  free(qd); free(od);
}

/* The copying append ([llmk] "KV-cache growth and greedy argmax": out = cache ++ new_vals): out receives
 * cache[0..cache_len) followed by new_vals rounded to the dtype; returns cache_len + n_new. */
int64_t orc_kv_append_copy(const void* cache, int64_t cache_len, const float* new_vals, int64_t n_new, int dtype,
                           void* out) {
  for (int64_t i = 0; i < cache_len; ++i) store(out, dtype, i, load(cache, dtype, i));
  for (int64_t i = 0; i < n_new; ++i) store(out, dtype, cache_len + i, (double)new_vals[i]);
  return cache_len + n_new;
}

/* ---- the decode step ------------------------------------------------------------------ */

typedef struct {
  int64_t vocab, d, n_layer, n_head, n_kv, head_dim, hidden;
  double eps, rope_base;
  int32_t rope_layout, w_dtype, kv_dtype;
} orc_shape;

/* Projections in the [in][out] layout; emb and out are [vocab][d]; gains fp32. */
typedef struct {
  const void* emb;
  const void* out;
  const float* norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const float* const* n1;
  const float* const* n2;
} orc_weights;

/* Per-layer K and V caches, each [max_seq][n_kv][hd] in kv_dtype, position-major
 * ([fwd] "The code": KVCache keeps one entry per position and layer); for ORC_Q8 each buffer holds the codes
 * [max_seq][n_kv][hd] followed by the scales [max_seq][n_kv] (orc_q8_row). */
typedef struct {
  void* const* k;
  void* const* v;
  int64_t max_seq;
} orc_cache;

/* One token through the decoder at position pos ([fwd] "What a forward step does" and "The code":
 * forward_token; [llmk] "How this composes into a decode step"):
 *   x = emb[token]
 *   per layer: h = rmsnorm(x, n1); q = wq^T h, k = wk^T h, v = wv^T h; RoPE(pos) on q and k;
 *              store k, v at pos (rounded to the cache dtype); attend over positions 0..pos;
 *              x += wo^T att; h = rmsnorm(x, n2); x += down^T (silu(gate^T h) * (up^T h))
 *   logits = out . rmsnorm(x, norm)
 * logits (fp32 [vocab]) and hidden (fp32 [n_layer][d], x after each layer; may be NULL) are written.
 * Returns 0, or -1 if pos is outside the cache. */
int orc_forward_token(const orc_shape* s, const orc_weights* w, const orc_cache* c, int64_t token, int64_t pos,
                      float* logits, float* hidden) {
  if (pos < 0 || pos >= c->max_seq || token < 0 || token >= s->vocab) return -1;
  const int64_t d = s->d, hd = s->head_dim, qd = s->n_head * hd, kvd = s->n_kv * hd, F = s->hidden;
  double* x = (double*)malloc(sizeof(double) * (size_t)d);
  double* h = (double*)malloc(sizeof(double) * (size_t)d);
  double* q = (double*)malloc(sizeof(double) * (size_t)qd);
  double* k = (double*)malloc(sizeof(double) * (size_t)kvd);
  double* v = (double*)malloc(sizeof(double) * (size_t)kvd);
  double* att = (double*)malloc(sizeof(double) * (size_t)qd);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  double* g = (double*)malloc(sizeof(double) * (size_t)F);
  double* u = (double*)malloc(sizeof(double) * (size_t)F);
  double* lg = (double*)malloc(sizeof(double) * (size_t)s->vocab);

  for (int64_t i = 0; i < d; ++i) x[i] = load(w->emb, s->w_dtype, token * d + i);
  for (int64_t l = 0; l < s->n_layer; ++l) {
    orc_rmsnorm(x, w->n1[l], d, s->eps, h);
    orc_gemv_t(w->wq[l], s->w_dtype, h, d, qd, q);
    orc_gemv_t(w->wk[l], s->w_dtype, h, d, kvd, k);
    orc_gemv_t(w->wv[l], s->w_dtype, h, d, kvd, v);
    orc_rope(q, s->n_head, hd, pos, s->rope_base, s->rope_layout);
    orc_rope(k, s->n_kv, hd, pos, s->rope_base, s->rope_layout);
    if (s->kv_dtype == ORC_Q8) {
      /* each head's row quantized into the cache, then attention over what the rows stand for */
      const int64_t codes_bytes = c->max_seq * kvd;
      for (int64_t g = 0; g < s->n_kv; ++g) {
        q8_store_row(c->k[l], codes_bytes, pos * s->n_kv + g, hd, k + g * hd);
        q8_store_row(c->v[l], codes_bytes, pos * s->n_kv + g, hd, v + g * hd);
      }
      double* kd = (double*)malloc(sizeof(double) * (size_t)((pos + 1) * kvd));
      double* vd = (double*)malloc(sizeof(double) * (size_t)((pos + 1) * kvd));
      q8_dequantize(c->k[l], codes_bytes, (pos + 1) * s->n_kv, hd, kd);
      q8_dequantize(c->v[l], codes_bytes, (pos + 1) * s->n_kv, hd, vd);
      orc_attend(q, kd, vd, ORC_F64, pos + 1, s->n_head, s->n_kv, hd, att);
      free(kd);
      free(vd);
    } else {
      for (int64_t i = 0; i < kvd; ++i) {
        store(c->k[l], s->kv_dtype, pos * kvd + i, k[i]);
        store(c->v[l], s->kv_dtype, pos * kvd + i, v[i]);
      }
      orc_attend(q, c->k[l], c->v[l], s->kv_dtype, pos + 1, s->n_head, s->n_kv, hd, att);
    }
    orc_gemv_t(w->wo[l], s->w_dtype, att, qd, d, y);
    for (int64_t i = 0; i < d; ++i) x[i] += y[i];
    orc_rmsnorm(x, w->n2[l], d, s->eps, h);
    orc_gemv_t(w->gate[l], s->w_dtype, h, d, F, g);
    orc_gemv_t(w->up[l], s->w_dtype, h, d, F, u);
    for (int64_t i = 0; i < F; ++i) g[i] = orc_silu(g[i]) * u[i];
    orc_gemv_t(w->down[l], s->w_dtype, g, F, d, y);
    for (int64_t i = 0; i < d; ++i) x[i] += y[i];
    if (hidden) for (int64_t i = 0; i < d; ++i) hidden[l * d + i] = (float)x[i];
  }
  orc_rmsnorm(x, w->norm, d, s->eps, h);
  orc_matvec(w->out, s->w_dtype, h, s->vocab, d, lg);
  for (int64_t r = 0; r < s->vocab; ++r) logits[r] = (float)lg[r];

  free(x); free(h); free(q); free(k); free(v); free(att); free(y); free(g); free(u); free(lg);
  return 0;
}

int orc_num_threads(void) { return omp_get_max_threads(); }
