/*
 * llmk.h -- C ABI of libllmk.so: one greedy decode step of a Llama/Qwen-style
 * grouped-query decoder, hand-written HIP for gfx950 (MI355X).
 *
 * Pages cited below (by title and section):
 *   [llmk]  "LLM inference kernels" (docs.algenta.ai, compute-and-kernel-primitives)
 *   [dops]  "decode-ops" (Hugging Face kernels page)
 *   [xpu]   "Inside the engine" (cajeta.dev, xpu/llm/inside)
 *   [fwd]   "The forward pass end to end: a Llama-style engine in 100 lines" (inferenceacademy.com)
 *
 * Conventions shared by every entry point
 *   - Every function that does work returns an int32 status from the vocabulary
 *     below. LLMK_OK means every check passed and the work is enqueued on `stream`
 *     (a hipStream_t; NULL is the null stream). Nothing is synchronised.
 *   - All checks run on the host before any HIP call and before any element is
 *     read ([llmk] "Guarantees": exact-length checks before any read). On any
 *     refusal nothing is enqueued and every output is left untouched.
 *   - Check order when several fail: null pointer or unknown enum (578), then a
 *     dimension < 1 or of the wrong sign (561), then a dimension > LLMK_MAX_DIM
 *     (564), then buffer lengths in argument order (the specific code), then
 *     value ranges (571-575), then workspace size (578).
 *   - A C pointer carries no length, so every buffer is passed with its element
 *     count; the pages' "claimed length vs real length" checks become a comparison
 *     of those counts.
 *   - Ownership: the caller allocates and owns all device memory (weights, K/V
 *     pool, workspace, outputs). The library allocates no device memory and keeps
 *     no pointer past the call ([xpu] "1. CausalLM": zero-allocation decode,
 *     every buffer sized at load).
 *   - Determinism: no float atomics; every reduction has a fixed order, so the
 *     same inputs on the same GPU give bit-identical outputs ([llmk] "Guarantees").
 *   - A launch failure reported by the HIP runtime after enqueue returns 579.
 *   - Pointers named `*_h` or documented as host are host memory; every other
 *     buffer pointer is device memory.
 */
#ifndef LLMK_H
#define LLMK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status vocabulary. 560-571 are the llmk page's codes with their meanings
 * ([llmk] "Status vocabulary and the shape checks (contract)"); the page reserves
 * 560-579 for this family and renumbers nothing, so the codes this library adds
 * take the free 572-579. 562/563 also serve as "first/second operand length
 * mismatch" for entry points the page does not have (rope, add_rmsnorm). */
enum {
  LLMK_OK = 560,                      /* every element of every output is defined */
  LLMK_EMPTY_DIMENSION = 561,         /* a required dimension was < 1 (or negative where 0 is allowed) */
  LLMK_A_LENGTH_MISMATCH = 562,       /* first operand's length != its dimension */
  LLMK_B_LENGTH_MISMATCH = 563,       /* second operand's length != its dimension */
  LLMK_DIMENSION_TOO_LARGE = 564,     /* a dimension exceeds LLMK_MAX_DIM */
  LLMK_CODE_OUT_OF_RANGE = 565,       /* not a code of this vocabulary (llmk_status_name's fallback) */
  LLMK_CACHE_LENGTH_MISMATCH = 566,   /* cache fill claimed != recorded */
  LLMK_NEW_LENGTH_MISMATCH = 567,     /* len(new_vals) != n_new */
  LLMK_LOGITS_LENGTH_MISMATCH = 568,  /* len(logits) != rows * n */
  LLMK_GEMV_A_LENGTH_MISMATCH = 569,  /* len(a) != m * n */
  LLMK_GEMV_X_LENGTH_MISMATCH = 570,  /* len(x) != m */
  LLMK_CACHE_CAPACITY_EXCEEDED = 571, /* the append would overrun the reserved buffer */
  LLMK_TOKEN_OUT_OF_RANGE = 572,      /* token id not in [0, vocab) */
  LLMK_POSITION_OUT_OF_RANGE = 573,   /* position < 0, or >= the RoPE table / max_seq */
  LLMK_HEAD_SHAPE_INVALID = 574,      /* a shape the kernels do not take: n_head % n_kv != 0, more than 8 query
                                         heads per K/V head, head_dim odd or > 256 (RoPE) or not a power of two
                                         in [2, 256] (attention, decode), widths not a whole number of vectors */
  LLMK_SLOT_OUT_OF_RANGE = 575,       /* K/V pool slot not in [0, n_slots) */
  LLMK_WEIGHT_LENGTH_MISMATCH = 576,  /* a model tensor's element count disagrees with the config */
  LLMK_OUTPUT_LENGTH_MISMATCH = 577,  /* an output buffer's element count disagrees with the shape */
  LLMK_INVALID_ARGUMENT = 578,        /* null pointer, unknown enum value, or workspace too small */
  LLMK_DEVICE_ERROR = 579             /* the HIP runtime reported an error */
};

/* Ceiling on every dimension: refuses byte counts passed as element counts
 * ([llmk] "Status vocabulary and the shape checks (contract)", "Guarantees"). */
#define LLMK_MAX_DIM (1LL << 24)
/* most sequences one batched decode step serves */
#define LLMK_MAX_BATCH 64

/* LLMK_Q8 is an int8 format: of the weights (llmk_config.w_dtype, llmk_quantize_q8; see "int8 weight packs"
 * below) and of the K/V pool (llmk_config.kv_dtype, llmk_kv_pool.dtype; see the pool below). */
typedef enum { LLMK_F32 = 0, LLMK_BF16 = 1, LLMK_Q8 = 2 } llmk_dtype;
/* Half-split pairs (j, j + hd/2) are the GPT-NeoX/Qwen3 convention ([llmk] "Two
 * gaps, not three"); interleaved pairs (2j, 2j+1) are the layout of [fwd] "The
 * code". [dops] "Method" supports both. */
typedef enum { LLMK_ROPE_HALF_SPLIT = 0, LLMK_ROPE_INTERLEAVED = 1 } llmk_rope_layout;
/* Storage of the seven per-layer projection matrices. LLMK_W_IN_OUT is the transposed-GEMV layout the
 * llmk page's decode driver uses (A[in][out], y = A^T x); LLMK_W_OUT_IN stores the same matrix output-major
 * (A^T, [out][in]), so every output is one contiguous row dot product. Both compute the same y; the
 * second streams faster and is what llmk_transpose produces, once, at load time. */
typedef enum { LLMK_W_IN_OUT = 0, LLMK_W_OUT_IN = 1 } llmk_weight_layout;

/* How llmk_decode_step / llmk_decode_steps run the step of one sequence. Both compute the same step
 * (the same arithmetic up to the order of fp32 sums). The persistent form needs bf16 weights in
 * LLMK_W_OUT_IN (or int8 packs with head_dim 64..256), a bf16 or fp32 K/V cache, and a device that holds
 * one of its workgroups per CU.
 *   LLMK_STEP_AUTO       the persistent kernel where it can run, else one kernel per operation
 *   LLMK_STEP_PER_OP     one kernel per operation: 5 per layer (q|k|v, attention, o, gate|up, down) + head
 *   LLMK_STEP_PERSISTENT one kernel per step, each operation waiting for the tagged outputs of the one
 *                        before it; refused (578) where it cannot run */
typedef enum { LLMK_STEP_AUTO = 0, LLMK_STEP_PER_OP = 1, LLMK_STEP_PERSISTENT = 2 } llmk_step_path;

/* ------------------------------------------------------------------------- */
/* Contract: host-only, no device needed ([llmk] "Status vocabulary and the    */
/* shape checks (contract)": four dimension checks, one per consumer).        */
/* ------------------------------------------------------------------------- */

/* Name of a status code, e.g. 562 -> "llmk_a_length_mismatch"; any other value
 * returns the name of 565, "llmk_code_out_of_range". Static string, never NULL. */
const char* llmk_status_name(int32_t code);

/* residual add: 561 if n < 1; 564 if n > LLMK_MAX_DIM; 562 if len_a != n; 563 if len_b != n.
 * [llmk] example: (6, 6, 6) -> 560; (6, 2, 6) -> 562. */
int32_t llmk_residual_dims_check(int64_t n, int64_t len_a, int64_t len_b);

/* K/V append: 561 if cache_len < 0 or n_new < 1 (an empty cache is allowed, an empty append is not,
 * [llmk] "Guarantees"); 564 if either exceeds LLMK_MAX_DIM; 566 if len_cache != cache_len;
 * 567 if len_new != n_new. */
int32_t llmk_kv_append_dims_check(int64_t cache_len, int64_t len_cache, int64_t n_new, int64_t len_new);

/* argmax: 561 if n < 1; 564 if n > LLMK_MAX_DIM; 568 if len_logits != n. */
int32_t llmk_argmax_dims_check(int64_t n, int64_t len_logits);

/* transposed GEMV: 561 if m < 1 or n < 1; 564 if m or n > LLMK_MAX_DIM; 569 if len_a != m*n;
 * 570 if len_x != m. */
int32_t llmk_gemv_dims_check(int64_t m, int64_t n, int64_t len_a, int64_t len_x);

/* ------------------------------------------------------------------------- */
/* Primitives (device buffers, caller's stream)                               */
/* ------------------------------------------------------------------------- */

/* Bytes of workspace llmk_gemv_t needs for an m x n matrix of dtype a_dtype (0 if none);
 * negative status if the shape itself is refused. */
int64_t llmk_gemv_t_workspace_bytes(int64_t m, int64_t n, int32_t a_dtype);

/* y = A^T x: y[j] = sum_i A[i*n + j] * x[i], A is m x n row-major ([in][out]), fp32 accumulation.
 * [llmk] "A parallel path for one frozen kernel's known-slow shape"; worked example
 * A = [[1,2,3],[4,5,6]], x = [1,1] -> y = [5,7,9].
 *   a      : device, m*n elements of a_dtype (LLMK_F32 or LLMK_BF16)
 *   x      : device fp32 [m];   y: device fp32 [n] (written)
 *   ws     : device workspace of len_ws bytes, >= llmk_gemv_t_workspace_bytes(m, n, a_dtype)
 * Codes: 578 (null / dtype / workspace), 561, 564, 569, 570, 577 (len_y != n). */
int32_t llmk_gemv_t(const void* a, int64_t len_a, int32_t a_dtype, const float* x, int64_t len_x,
                    int64_t m, int64_t n, float* y, int64_t len_y, void* ws, int64_t len_ws, void* stream);

/* y = W x (untransposed, row dots): y[r] = sum_c W[r*cols + c] * x[c]; the output head's form
 * ([llmk] "A parallel path...": the untransposed lm_head; [fwd] "The code": matvec).
 * Codes: 578, 561, 564, 569 (len_w != rows*cols), 570 (len_x != cols), 577 (len_y != rows). */
int32_t llmk_gemv(const void* w, int64_t len_w, int32_t w_dtype, const float* x, int64_t len_x,
                  int64_t rows, int64_t cols, float* y, int64_t len_y, void* stream);

/* out[i] = a[i] + b[i], fp32 ([llmk] "Residual add"). out may alias a or b.
 * Codes: 578, 561, 564, 562, 563, 577 (len_out != n). */
int32_t llmk_residual_add(const float* a, int64_t len_a, const float* b, int64_t len_b, int64_t n,
                          float* out, int64_t len_out, void* stream);

/* For each of `rows` rows of width n: if x != NULL, residual += x (in place, fp32); then
 * h = residual * (mean(residual^2) + eps)^(-1/2) * gain, with the square sum in fp32
 * ([dops] "Usage", "Method"; [fwd] "The code": rmsnorm). x == NULL gives the plain norm.
 *   residual: device fp32 [rows*n] (read, and written when x != NULL); x: device fp32 [rows*n] or NULL
 *   gain: device fp32 [n]; h: device fp32 [rows*n] (written; may not alias residual)
 * Codes: 578 (null residual/gain/h, eps <= 0 or not finite), 561, 564, 562 (len_r != rows*n),
 * 563 (x given and len_x != rows*n), 576 (len_g != n), 577 (len_h != rows*n). */
int32_t llmk_add_rmsnorm(float* residual, int64_t len_r, const float* x, int64_t len_x,
                         const float* gain, int64_t len_g, int64_t rows, int64_t n, float eps,
                         float* h, int64_t len_h, void* stream);

/* out[i] = silu(gate[i]) * up[i], silu(z) = z / (1 + e^-z) ([dops] "Usage"; [fwd] "The code").
 * Codes: 578, 561, 564, 562, 563, 577. */
int32_t llmk_silu_mul(const float* gate, int64_t len_gate, const float* up, int64_t len_up, int64_t n,
                      float* out, int64_t len_out, void* stream);

/* RoPE cos/sin table: table[(p*(hd/2) + j)*2 + {0,1}] = {cos, sin}(p * base^(-2j/hd)) for
 * p in [0, max_pos), j in [0, hd/2); angles and trig in fp64, stored fp32 ([dops] "Method":
 * angle pairs in f64; [llmk] "The hot loop doesn't call kv_cache_append_flat": one shared table
 * sized to the longest sequence). len_table must be max_pos * head_dim.
 * Codes: 578 (null, base <= 1 or not finite), 561, 564, 574 (odd head_dim or > 256), 577. */
int32_t llmk_rope_table_init(float* table, int64_t len_table, int64_t max_pos, int64_t head_dim,
                             double base, void* stream);

/* In-place rotary embedding of q [rows][n_q_heads][hd] and k [rows][n_k_heads][hd]; row r is at
 * position pos[r], read on the device ([dops] "Usage": rope(q, k, pos) in place), so a step whose
 * positions live on the device needs no host round trip. layout selects half-split or interleaved pairs.
 * k may be NULL with n_k_heads == 0.
 *   pos: device int32 [rows] (len_pos elements). The host cannot see device positions: a row whose
 *        position is outside [0, max_pos) has no table row and is left unchanged.
 * Codes: 578 (null q/table/pos, layout, k NULL with n_k_heads > 0), 561 (rows, n_q_heads, head_dim,
 * max_pos < 1, or n_k_heads < 0), 564, 574 (odd hd or > 256), 562 (len_q), 563 (len_k), 576 (len_table !=
 * max_pos*hd), 577 (len_pos != rows). */
int32_t llmk_rope(float* q, int64_t len_q, float* k, int64_t len_k, int64_t rows, int64_t n_q_heads,
                  int64_t n_k_heads, int64_t head_dim, const int32_t* pos, int64_t len_pos, const float* table,
                  int64_t len_table, int64_t max_pos, int32_t layout, void* stream);

/* In-place append into one reserved flat cache buffer: cache[cache_len + i] = round(new_vals[i]) for
 * i in [0, n_new), rounded to the cache dtype (fp32 -> bf16 round-to-nearest-even, NaN kept).
 * Existing content is never copied ([llmk] "KV-cache growth and greedy argmax" and "The hot loop
 * doesn't call kv_cache_append_flat": the reserved-capacity, in-place append). llmk_kv_append is the
 * same append into one (layer, slot, K or V) buffer of a pool.
 *   cache     : device buffer of `capacity` elements of `dtype`
 *   cache_len : claimed filled length; len_cache: the caller's record of it (566 if different)
 *   new_len_h : host int64, receives cache_len + n_new on success (may be NULL)
 * Codes: 578, 561 (capacity < 1, cache_len < 0, n_new < 1), 564, 566, 567, 571 (cache_len + n_new >
 * capacity). Worked example: cache [0..5], new [100,101,102] -> 9 elements, n = 9. */
int32_t llmk_kv_append_flat(void* cache, int64_t capacity, int32_t dtype, int64_t cache_len, int64_t len_cache,
                            const float* new_vals, int64_t len_new, int64_t n_new, int64_t* new_len_h, void* stream);

/* Bytes of workspace llmk_gqa_attend_flat and llmk_gqa_attend need. */
int64_t llmk_gqa_attend_workspace_bytes(int64_t ctx_len, int64_t n_head, int64_t head_dim);

/* Grouped-query decode attention for one query position over a cache of ctx_len positions:
 * for head h with K/V head g = h / (n_head / n_kv): s_t = q_h . K[t][g] / sqrt(hd), w = softmax(s),
 * out_h = sum_t w_t V[t][g] ([fwd] "The code": forward_token's attention loop). The context is
 * split into chunks whose partial (max, sum, output) are merged by log-sum-exp ([xpu] "1. CausalLM":
 * flash attention split across the context and reduced).
 *   q: device fp32 [n_head][hd]; k_cache, v_cache: device [>= ctx_len][n_kv][hd] of kv_dtype
 *   len_cache: elements in each of k_cache and v_cache; out: device fp32 [n_head][hd]
 *   ws: device workspace of len_ws >= llmk_gqa_attend_workspace_bytes bytes (no clearing needed)
 * Codes: 578, 561, 564, 574 (n_head % n_kv != 0, n_head / n_kv > 8, hd not a power of two in [2, 256]),
 * 562 (len_q), 563 (len_cache < ctx_len*n_kv*hd), 577 (len_out), 578 (workspace short, caches not
 * 16-byte aligned). llmk_gqa_attend is the same attention over one (layer, slot) of a pool. */
int32_t llmk_gqa_attend_flat(const float* q, int64_t len_q, const void* k_cache, const void* v_cache,
                             int64_t len_cache, int32_t kv_dtype, int64_t ctx_len, int64_t n_head, int64_t n_kv,
                             int64_t head_dim, float* out, int64_t len_out, void* ws, int64_t len_ws, void* stream);

/* Bytes of workspace llmk_argmax needs. */
int64_t llmk_argmax_workspace_bytes(int64_t rows, int64_t n);

/* Greedy argmax per row: token[r] = the lowest i with logits[r*n + i] equal to the row maximum,
 * logit[r] = that maximum ([llmk] "KV-cache growth and greedy argmax": first matching id on ties;
 * [dops] "Correctness": exact against torch.argmax including ties). NaN counts as larger than every
 * number and the first NaN wins (numpy/torch convention). +0.0 and -0.0 compare equal.
 *   token: device int32 [rows]; logit: device fp32 [rows] (may be NULL)
 * Codes: 578, 561, 564, 568 (len_logits != rows*n), 578 (workspace). */
int32_t llmk_argmax(const float* logits, int64_t len_logits, int64_t rows, int64_t n, int32_t* token,
                    float* logit, void* ws, int64_t len_ws, void* stream);

/* llmk_argmax for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same result, with the per-block partials and tickets in a
 * fixed scratch array the library holds on each GPU (about 129 KiB, kept until the process ends) instead of
 * a caller workspace. The call allocates nothing. Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (different streams, or host threads) race and must be serialised by the caller.
 *   token: device int32 [rows]; logit: device fp32 [rows] (may be NULL)
 * Codes: 578 (null logits/token), 561, 564, 568 (len_logits != rows*n), 564 (rows >
 * LLMK_ARGMAX_NOALLOC_MAX_ROWS), 579 (the array's address could not be obtained). */
#define LLMK_ARGMAX_NOALLOC_MAX_ROWS 256
int32_t llmk_argmax_noalloc(const float* logits, int64_t len_logits, int64_t rows, int64_t n, int32_t* token,
                            float* logit, void* stream);

/* Survivors llmk_sample holds: top_k after clamping to n (1 at temperature 0); rows one call takes. */
#define LLMK_SAMPLE_MAX_K 1024
#define LLMK_SAMPLE_MAX_ROWS 65535

/* Workspace bytes llmk_sample needs for these sizes (0: none), or -status for invalid sizes. */
int64_t llmk_sample_workspace_bytes(int64_t rows, int64_t n, float temperature, int32_t top_k);

/* One sampled token per row of logits ([dops] "Method" sets the sequence of the cuts and how ties rank).
 * Candidates: the top_k largest logits, equal logits ranked lower index first. Their weights: softmax of
 * logit / temperature over the candidates. Walking the candidates in rank order, one stays while the total
 * weight of those ranked ahead of it is under top_p, so the first always stays; the row's token is the first
 * staying candidate at which the running sum of the staying weights, taken as a fraction of their total,
 * passes u[r]. temperature 0 is greedy (the lowest index
 * holding the row maximum). A NaN logit counts as -inf and -0 as +0; a draw below 0 or NaN counts as 0, a
 * draw of 1 or more takes the last kept survivor with mass. The same row and draw always give the same
 * token (no float atomics).
 *   logits: device fp32 [rows][n]; u: device fp32 [rows], one draw in [0, 1) per row; token: device int32
 *   [rows]. top_k <= 0 or >= n means n. ws: device scratch of len_ws >= llmk_sample_workspace_bytes bytes,
 *   16-byte aligned (may be NULL when that is 0); its contents need no clearing and are dead after the call.
 * Codes: 578 (null logits/u/token), 561, 564, 568 (len_logits != rows*n), 563 (len_u != rows), 578
 * (temperature < 0 or NaN, top_p not in (0, 1]), 564 (survivors min(top_k, n) > LLMK_SAMPLE_MAX_K at a
 * temperature above 0, or rows > LLMK_SAMPLE_MAX_ROWS), 578 (workspace missing, short or misaligned). */
int32_t llmk_sample(const float* logits, int64_t len_logits, int64_t rows, int64_t n, float temperature,
                    int32_t top_k, float top_p, const float* u, int64_t len_u, int32_t* token, void* ws,
                    int64_t len_ws, void* stream);

/* ------------------------------------------------------------------------- */
/* Model, K/V pool and the decode step                                        */
/* ------------------------------------------------------------------------- */

/* Decoder shape and numerics. head_dim is independent of d (Qwen3 shapes have n_head*head_dim != d). */
typedef struct {
  int64_t vocab, d, n_layer, n_head, n_kv, head_dim, hidden, max_seq;
  double eps;          /* RMSNorm epsilon, inside the mean ([fwd] "The code": rmsnorm) */
  double rope_base;    /* RoPE base (1e4 for the toy decoder, 1e6 Qwen3-shaped, 5e5 Llama-3-shaped) */
  int32_t rope_layout; /* llmk_rope_layout */
  int32_t w_dtype;     /* llmk_dtype of every weight matrix and the embedding table; LLMK_Q8: the seven
                          projections and the output head are q8 packs and the embedding table is bf16 */
  int32_t kv_dtype;    /* llmk_dtype of the K/V pool; LLMK_Q8: int8 rows (llmk_kv_pool), head_dim a multiple of
                          16 (574), decode steps run one kernel per operation (LLMK_STEP_PERSISTENT: 578) */
  int32_t w_layout;    /* llmk_weight_layout of the seven per-layer projections */
  int32_t step_path;   /* llmk_step_path */
  int32_t test_flags;  /* 0 in normal use; LLMK_TEST_* bits exercise error paths in tests */
} llmk_config;

/* llmk_config.test_flags: LLMK_TEST_WAIT_GIVE_UP makes every cross-workgroup wait of the persistent step
 * wait for a hand-off tag that no workgroup writes, so the first wait runs into its bounded-wait limit
 * (200 ms), every workgroup then stops waiting and exits, and the call returns 579. Only the persistent
 * form has such waits; the per-operation form ignores the flag. For tests of the failure path only. */
#define LLMK_TEST_WAIT_GIVE_UP 1

/* A device tensor and its element count. */
typedef struct {
  const void* ptr;
  int64_t len;
} llmk_tensor;

/* Per-layer tensors, in this order, LLMK_LAYER_TENSORS per layer. With LLMK_W_IN_OUT the projections are
 * in the transposed layout A[in][out] (y = A^T x), as the llmk page's decode driver uses them:
 *   wq [d][H*hd]  wk [d][Hkv*hd]  wv [d][Hkv*hd]  wo [H*hd][d]
 *   w_gate [d][F]  w_up [d][F]  w_down [F][d]  (w_dtype)
 * With LLMK_W_OUT_IN each of these seven is stored transposed ([out][in]); element counts are the same.
 *   g_attn [d]  g_ffn [d]  (fp32 RMSNorm gains) */
enum { LLMK_WQ = 0, LLMK_WK, LLMK_WV, LLMK_WO, LLMK_WGATE, LLMK_WUP, LLMK_WDOWN, LLMK_GATTN, LLMK_GFFN,
       LLMK_LAYER_TENSORS };

typedef struct {
  llmk_tensor emb;         /* [vocab][d], w_dtype */
  llmk_tensor w_out;       /* [vocab][d], w_dtype (untransposed output head) */
  llmk_tensor g_final;     /* [d] fp32 */
  llmk_tensor rope_table;  /* fp32 [max_seq][hd/2][2] from llmk_rope_table_init(max_seq, hd, rope_base) */
  const llmk_tensor* layers; /* host array [n_layer * LLMK_LAYER_TENSORS] */
} llmk_model;

/* Paged K/V blocks ([xpu] "3. The K/V cache and the block store": the cache is paged in fixed blocks of
 * block_tokens positions, shared between sequences by reference count with copy-on-write, and a full pool
 * refuses the append). With llmk_kv_pool.pages set, each layer buffer is a store of n_blocks blocks, and
 * position p of slot s, K/V head g, element i sits at
 *   (b * block_tokens + p % block_tokens) * n_kv * head_dim + g * head_dim + i,
 *   b = table[s * max_blocks + p / block_tokens],
 * so each layer buffer holds n_blocks * block_tokens * n_kv * head_dim elements. One block id names the same
 * positions in every layer's K and V buffer. capacity stays the most positions one slot may hold.
 * The caller allocates every array and the library keeps them consistent: before an entry point writes
 * positions of a slot it reserves them, in slot order and then block order:
 *   - a table entry of -1 takes the lowest-numbered free block;
 *   - an entry whose block other slots also hold (refcount > 1) is copied first: the lowest-numbered free
 *     block receives the whole block (every layer, K and V), the old block's refcount drops by one and the
 *     entry moves to the copy (copy-on-write);
 *   - when the free blocks cannot cover every block the call needs, it returns 571 and changes nothing;
 *   - when the stream is being captured into a graph and the reservation needs device work (a copy or a
 *     table write), it returns 578: a captured graph would repeat that work on every replay (reserve ahead
 *     with llmk_kv_reserve instead).
 * These codes apply to every entry point that writes a paged pool (decode steps single and batched,
 * prefill, llmk_kv_append); their other checks run first. The device table is written by the library (stream-ordered kernels) as entries change; entries that were
 * never reserved are never read. A block's refcount is the number of table entries that hold it. */
typedef struct {
  int64_t block_tokens;    /* positions per block: a power of two in [64, 65536] */
  int64_t n_blocks;        /* blocks in each layer buffer, at most LLMK_MAX_DIM */
  int64_t max_blocks;      /* table entries per slot: ceil(capacity / block_tokens) */
  int32_t* table;          /* device int32 [n_slots][max_blocks] */
  int32_t* table_h;        /* host int32 [n_slots][max_blocks]: the block of each entry, -1 for none */
  int32_t* refcount_h;     /* host int32 [n_blocks] */
  int64_t n_free;          /* blocks with refcount 0 */
} llmk_kv_pages;

/* Slot-indexed device K/V pool ([xpu] "3. The K/V cache and the block store": one K and one V
 * buffer per layer, slot s at element s * plane). Without pages (pages == NULL), layer l's K buffer holds
 * n_slots * capacity * n_kv * head_dim elements; position p of slot s, K/V head g, element i sits at
 *   s * plane + p * n_kv * head_dim + g * head_dim + i,   plane = capacity * n_kv * head_dim.
 * With pages, positions reach their blocks through the block table (llmk_kv_pages above).
 * int8 pool (dtype LLMK_Q8; the pages name int8 K/V caches without a format, [dops] opening paragraph,
 * [xpu] "1. CausalLM", so the format is this library's): every (position, K/V head) row of head_dim values
 * is stored as head_dim int8 codes and one fp32 scale, s = max|x| / 127, code = rint(x / s) (both fp32
 * divisions, ties to even) clamped to [-127, 127] (a zero row: s = 0, codes 0); the row stands for code * s.
 * Each layer buffer holds the codes of every cache row at the element offsets above (one byte each), then,
 * from byte rows * n_kv * head_dim on, the scales fp32 [rows][n_kv] (rows = n_slots * capacity, or
 * n_blocks * block_tokens with pages): the scale of (cache row r, K/V head g) at index r * n_kv + g. head_dim
 * is a multiple of 16. The decode steps (single, batched), prefill and llmk_gqa_attend take int8 pools;
 * llmk_kv_append (a flat append of elements) refuses them.
 * slot_len_h records how many positions each slot holds; decode steps check it (566) and advance it.
 * len_k_h / len_v_h, when given, record the filled elements of every (layer, slot) K and V buffer, the
 * flat cache lengths llmk_kv_append checks and advances ([llmk] "KV-cache growth and greedy argmax":
 * cache_len -> cache_len + n_new); decode steps and prefill set them to positions * n_kv * head_dim for
 * every layer of the slots they advance. */
typedef struct {
  void* const* k;          /* host array [n_layer] of device pointers */
  void* const* v;          /* host array [n_layer] of device pointers */
  int64_t n_layer, n_slots, capacity, n_kv, head_dim;
  int32_t dtype;           /* llmk_dtype */
  int64_t* slot_len_h;     /* host array [n_slots] */
  int64_t* len_k_h;        /* host array [n_layer][n_slots] or NULL */
  int64_t* len_v_h;        /* host array [n_layer][n_slots] or NULL */
  llmk_kv_pages* pages;    /* NULL: contiguous slots */
} llmk_kv_pool;

/* Validate a pool descriptor and mark every slot empty: slot_len_h, and len_k_h / len_v_h when given, are
 * set to 0 ([llmk] "The hot loop doesn't call kv_cache_append_flat": the cache is reserved once at its full
 * capacity, then filled in place). With pages, every table_h entry becomes -1, every refcount 0 and n_free
 * n_blocks. Host only; the device buffers (and the device table) are not touched.
 * Codes: 578 (null pool, k, v, slot_len_h or a layer buffer, unknown dtype, buffers not 16-byte aligned;
 * pages with a null table, table_h or refcount_h, block_tokens not a power of two in [64, 65536],
 * max_blocks != ceil(capacity / block_tokens)), 561 (n_layer, n_slots, capacity, n_kv, head_dim or n_blocks
 * < 1), 564 (> LLMK_MAX_DIM, or n_slots * max_blocks > LLMK_MAX_DIM), 574 (dtype LLMK_Q8 and head_dim not a
 * multiple of 16, checked after the dimensions). The pages are checked after the rest. */
int32_t llmk_kv_pool_init(llmk_kv_pool* pool);

/* llmk_kv_append_flat on buffer `which` (0: K, 1: V) of `layer` for sequence `slot`: the slot's region is a
 * flat cache of capacity * n_kv * head_dim elements whose recorded fill is len_k_h / len_v_h[layer * n_slots
 * + slot]. cache_len is the caller's claim of that fill and n_new the elements appended (a decode token
 * appends n_kv * head_dim, one position). On success the record becomes cache_len + n_new, *new_len_h gets
 * it and *elem_offset_h gets the element offset of the first written element in the layer buffer,
 * slot * plane + cache_len ([xpu] "3. The K/V cache and the block store": slot s at s * plane).
 * With pages the positions the new elements fall in are reserved first (llmk_kv_reserve's rules), element e
 * of the slot's flat cache goes to position e / (n_kv * head_dim) through the table, and *elem_offset_h is
 * the offset of the first written element.
 *   new_vals: device fp32 [len_new]; new_len_h, elem_offset_h: host int64 (each may be NULL)
 * Codes: 578 (null pool / new_vals, len_k_h or len_v_h NULL, which not 0 or 1, an int8 pool, layer not in
 * [0, n_layer)),
 * 561 (cache_len < 0, n_new < 1), 564, 575 (slot), 566 (cache_len != recorded fill), 567 (len_new != n_new),
 * 571 (cache_len + n_new > capacity * n_kv * head_dim, or, with pages, too few free blocks), 578 (with
 * pages: the stream is being captured and the reserve has device work). */
int32_t llmk_kv_append(llmk_kv_pool* pool, int64_t layer, int64_t slot, int32_t which, int64_t cache_len,
                       const float* new_vals, int64_t len_new, int64_t n_new, int64_t* new_len_h,
                       int64_t* elem_offset_h, void* stream);

/* llmk_gqa_attend_flat over positions [0, ctx_len) of one (layer, slot) of a pool ([fwd] "The code": the
 * attention over the cached keys and values; [xpu] "3. The K/V cache and the block store").
 *   q: device fp32 [n_head][head_dim]; out: device fp32 [n_head][head_dim]; ws as for llmk_gqa_attend_flat
 * Codes: 578 (null, layer not in [0, n_layer)), 561 (ctx_len or n_head < 1), 564, 575 (slot), 574 (as
 * llmk_gqa_attend_flat with the pool's n_kv and head_dim), 562 (len_q), 577 (len_out), 573 (ctx_len >
 * capacity, or, with pages, a position of [0, ctx_len) without a block), 566 (len_k_h / len_v_h given and
 * either records fewer than ctx_len positions), 578 (workspace). With pages the kernel reads through the
 * table. */
int32_t llmk_gqa_attend(const float* q, int64_t len_q, const llmk_kv_pool* pool, int64_t layer, int64_t slot,
                        int64_t ctx_len, int64_t n_head, float* out, int64_t len_out, void* ws, int64_t len_ws,
                        void* stream);

/* Element offset of (slot, pos, kv_head) in each layer buffer of the pool (closed forms above; with pages,
 * through the host mirror of the table).
 * Codes: 578, 575 (slot), 573 (pos not in [0, capacity), or, with pages, its block not reserved),
 * 574 (kv_head not in [0, n_kv)). */
int32_t llmk_kv_slot_offset(const llmk_kv_pool* pool, int64_t slot, int64_t pos, int64_t kv_head,
                            int64_t* offset_h);

/* Paged pools only: make positions [pos_begin, pos_end) of `slot` writable by the rules above (fresh blocks
 * for entries of -1, copies for shared blocks) ([xpu] "2. The scheduler: continuous batching": the K/V
 * reserve phase of a step). Every entry point that writes positions does this itself; a caller reserves
 * ahead to keep later calls free of device work, e.g. before capturing a graph of decode steps.
 * The block copies and table writes are enqueued on `stream`.
 * Codes: 578 (null, pool without pages, or the stream is being captured and the reserve has device work),
 * 561 (pos_begin < 0 or pos_end <= pos_begin), 564, 575 (slot), 571 (pos_end > capacity, or too few free
 * blocks: nothing changed). */
int32_t llmk_kv_reserve(llmk_kv_pool* pool, int64_t slot, int64_t pos_begin, int64_t pos_end, void* stream);

/* Paged pools only: slot dst takes the first n_pos positions of slot src by sharing the blocks that hold
 * them (each refcount + 1; [xpu] "3. The K/V cache and the block store": sequences forked from a common
 * prefix share its blocks). dst must be empty (no positions, no blocks). Afterwards slot_len_h[dst] = n_pos
 * and, when given, dst's len_k_h / len_v_h records are n_pos * n_kv * head_dim. The first write of either
 * slot into a shared block copies it. dst's table row is written on `stream`.
 * Codes: 578 (null, pool without pages, src == dst), 561 (n_pos < 1), 564, 575 (src or dst),
 * 566 (n_pos > slot_len_h[src], or dst not empty). */
int32_t llmk_kv_fork(llmk_kv_pool* pool, int64_t src, int64_t dst, int64_t n_pos, void* stream);

/* Paged pools only: drop every block of `slot` (refcount - 1 each; a block reaching 0 is free), clear its
 * table row (host mirror) and mark it empty (slot_len_h and, when given, its len_k_h / len_v_h records 0)
 * ([xpu] "2. The scheduler: continuous batching": completions free blocks). Host only.
 * Codes: 578 (null, pool without pages), 575 (slot). */
int32_t llmk_kv_release(llmk_kv_pool* pool, int64_t slot);

/* Paged pools only: the admission rule ([xpu] "2. The scheduler: continuous batching", "Admission": the free
 * blocks must cover the request's whole uncached suffix plus one block of decode headroom per layer that is
 * not windowed). A block here spans every layer (no layer is windowed), so the headroom is one block:
 *   *admit_h = n_free >= ceil(n_uncached / block_tokens) + 1.
 * Codes: 578 (null, pool without pages), 561 (n_uncached < 0), 564. */
int32_t llmk_kv_admit(const llmk_kv_pool* pool, int64_t n_uncached, int32_t* admit_h);

/* Bytes of workspace a decode call needs for `batch` rows (negative status if cfg is refused). batch 1
 * covers llmk_decode_step / llmk_decode_steps and, when the config allows the batched path, the batched
 * entry points with one row; batch 2..LLMK_MAX_BATCH needs bf16 weights in LLMK_W_OUT_IN (else -578). */
int64_t llmk_decode_workspace_bytes(const llmk_config* cfg, int64_t batch);

/* One decode step of one sequence ([fwd] "What a forward step does"; [llmk] "How this composes into
 * a decode step"): x = emb[token]; per layer h = rmsnorm(x) g_attn; q|k|v = h W; RoPE(pos) on q, k;
 * append k, v to the slot at pos; grouped-query attention over positions 0..pos; x += att Wo;
 * h = rmsnorm(x) g_ffn; x += (silu(h Wgate) * (h Wup)) Wdown; then logits = W_out rmsnorm(x) g_final
 * and the greedy token ([xpu] "1. CausalLM": the fused tail reads back one integer).
 *   token, pos : the input token and its position; pos must equal pool->slot_len_h[slot] (566)
 *   logits     : device fp32 [vocab] or NULL;  token_out: device int32 [1]
 *   hidden     : device fp32 [n_layer][d] (the residual after each layer) or NULL
 * On success pool->slot_len_h[slot] becomes pos + 1.
 * The persistent form hands activations between workgroups through bounded waits; there the call waits
 * for the step to finish and returns 579 if a wait gave up (its outputs are then undefined). When `stream`
 * is being captured into a graph it cannot wait, and such a failure is not reported by this call.
 * Codes: 578, 561/564/574 (config), 576 (model tensor lengths), 575, 572, 573 (pos < 0 or >= max_seq),
 * 566, 571 (pos >= capacity), 568 (len_logits != vocab), 577 (len_hidden), 578 (workspace), then the paged
 * reservation's 571 / 578, 579. */
int32_t llmk_decode_step(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                         int64_t token, int64_t pos, float* logits, int64_t len_logits, int32_t* token_out,
                         float* hidden, int64_t len_hidden, void* ws, int64_t len_ws, void* stream);

/* n_steps greedy steps of one sequence: step i consumes the token at position pos0 + i (token0 for
 * i = 0, else the previous step's output, fed back on the device) and writes its greedy token to
 * tokens_out[i]. The step's launch sequence is captured once into a HIP graph and replayed, and the
 * host reads nothing between steps ([xpu] "4. The pipelined decode"). Returns after `stream` has
 * finished the steps, so the graph can be released.
 *   tokens_out: device int32 [n_steps] (len_tokens elements)
 * Codes: as llmk_decode_step, plus 561/564 for n_steps and 571 if pos0 + n_steps > capacity,
 * 573 if pos0 + n_steps > max_seq. On success slot_len_h[slot] = pos0 + n_steps. */
int32_t llmk_decode_steps(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                          int64_t token0, int64_t pos0, int64_t n_steps, int32_t* tokens_out, int64_t len_tokens,
                          void* ws, int64_t len_ws, void* stream);

/* As llmk_decode_steps, with the sampling exit in place of greedy at the end of every step (llmk_sample's
 * rule exactly; [dops] "Method"): step i samples its token from its logits with the uniform draws[i],
 * writes it to tokens_out[i] and feeds it to step i + 1, all inside the captured loop.
 *   draws: device fp32 [n_steps] (len_draws elements), the caller's uniforms in [0, 1)
 *   temperature >= 0 (0: greedy), top_k <= 0 or >= vocab: no cut, 0 < top_p <= 1
 *   sample_ws: device scratch of len_sample_ws >= llmk_sample_workspace_bytes(1, vocab, temperature, top_k)
 *   bytes, 16-byte aligned (may be NULL where that is 0); ws as for llmk_decode_steps
 * Codes: as llmk_decode_steps (578 also for a NULL draws), then 563 (len_draws != n_steps), 578 (temperature,
 * top_p), 564 (more than LLMK_SAMPLE_MAX_K survivors), 578 (sample_ws too small or misaligned). */
int32_t llmk_decode_steps_sampled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                  int64_t token0, int64_t pos0, int64_t n_steps, float temperature, int32_t top_k,
                                  float top_p, const float* draws, int64_t len_draws, int32_t* tokens_out,
                                  int64_t len_tokens, void* ws, int64_t len_ws, void* sample_ws,
                                  int64_t len_sample_ws, void* stream);

/* One decode step of `batch` sequences at once ([xpu] "5. The batched decode": every weight row is read
 * once for all rows of the batch; the projections run as bf16 matrix-core GEMMs with each fp32 activation
 * carried as a bf16 hi + lo pair, fp32 accumulation). Row r is sequence slot slots_h[r] with input token
 * tokens_h[r] at position pos_h[r]; each row computes exactly llmk_decode_step's step for its sequence
 * (its own context length, its own K/V append).
 *   slots_h, tokens_h, pos_h: host int64 [batch]; slots distinct
 *   logits    : device fp32 [batch][vocab] or NULL (len_logits = batch * vocab)
 *   tokens_out: device int32 [batch] (len_tokens = batch)
 *   hidden    : device fp32 [batch][n_layer][d] or NULL (len_hidden = batch * n_layer * d)
 * Needs bf16 weights in LLMK_W_OUT_IN. On success slot_len_h[slots_h[r]] = pos_h[r] + 1 for every row.
 * Codes, in order: 578 (null), config codes, 561 (batch < 1), 564 (batch > LLMK_MAX_BATCH), 578 (model
 * tensors), 576, pool 578/561/564, 578 (alignment, or weights not bf16 LLMK_W_OUT_IN), then over all
 * rows: 575 (slot), 578 (a slot repeated), 572 (token), 573 (pos), 566 (pos != slot length), 571
 * (capacity); then 568 (len_logits), 577 (len_tokens, len_hidden), 578 (workspace). */
int32_t llmk_decode_step_batch(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t batch,
                               const int64_t* slots_h, const int64_t* tokens_h, const int64_t* pos_h, float* logits,
                               int64_t len_logits, int32_t* tokens_out, int64_t len_tokens, float* hidden,
                               int64_t len_hidden, void* ws, int64_t len_ws, void* stream);

/* n_steps greedy batched steps: row r's step i consumes the token at position pos0_h[r] + i (tokens0_h[r]
 * for i = 0, else its previous output, fed back on the device) and writes its greedy token to
 * tokens_out[i * batch + r]. One step is captured into a HIP graph and replayed; returns after `stream`
 * has finished. tokens_out: device int32 [n_steps][batch] (len_tokens = n_steps * batch).
 * Codes: as llmk_decode_step_batch (without the logits/hidden checks), plus 561/564 for n_steps; 573 and
 * 571 take pos0 + n_steps. On success slot_len_h[slots_h[r]] = pos0_h[r] + n_steps. */
int32_t llmk_decode_steps_batch(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t batch,
                                const int64_t* slots_h, const int64_t* tokens0_h, const int64_t* pos0_h,
                                int64_t n_steps, int32_t* tokens_out, int64_t len_tokens, void* ws, int64_t len_ws,
                                void* stream);

/* Workspace bytes llmk_prefill needs for an n-token prompt (the row buffers, projection partials, logits and
 * hidden states of one chunk), or -status: the config's check code, 561/564 for n, 578 where the
 * batched path cannot run (weights not bf16 output-major). */
int64_t llmk_prefill_workspace_bytes(const llmk_config* cfg, int64_t n);

/* Prefill of n prompt tokens into one slot ([xpu] "1. CausalLM: the forward path": a prompt chunk is a batch
 * of rows through the batched projections, and decode is the one-token chunk of the same step). Positions
 * pos0 .. pos0 + n - 1 of `slot`, in chunks of up to 256 rows: per layer the chunk's rows go through the
 * q|k|v projection together (a tiled matrix-core GEMM, each weight tile serving every row), then all rows'
 * k (rotated) and v are written to the cache, then row i attends over positions 0 .. pos0 + i of the slot
 * (causal), then o, gate|up and down the same way; the head's logits of every row give its greedy token. The result equals n decode steps fed tokens_h[0..n) one by one.
 *   tokens_h: host int64 [n]; tokens_out: device int32 [n], the greedy token after each position;
 *   logits (optional, NULL to skip): device fp32 [vocab] of the last position; hidden (optional): device
 *   fp32 [n_layer][d], the residual after every layer at the last position. ws: device scratch of len_ws >=
 *   llmk_prefill_workspace_bytes(cfg, n) bytes, 256-byte aligned, contents dead after the call.
 * Codes, in order: 578 (null cfg/model/pool/tokens_h/tokens_out/ws), the config's check code, 561/564 (n),
 * model and pool checks as llmk_decode_step, 578 (weights not bf16 output-major, or misaligned), 575 (slot),
 * 572 (a token), 573 (pos0 < 0 or pos0 + n > max_seq), 566 (pos0 != slot length), 571 (pos0 + n > capacity),
 * 577 (len_tokens != n), 568 (len_logits != vocab), 577 (len_hidden != n_layer * d), 578 (workspace).
 * On success slot_len_h[slot] = pos0 + n; the call returns once the work is queued on `stream`. */
int32_t llmk_prefill(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                     const int64_t* tokens_h, int64_t n, int64_t pos0, int32_t* tokens_out, int64_t len_tokens,
                     float* logits, int64_t len_logits, float* hidden, int64_t len_hidden, void* ws, int64_t len_ws,
                     void* stream);

/* Measurement aid (not on the prefill path): llmk_prefill (logits and hidden not returned) with a HIP event
 * recorded on `stream` at every boundary between its phases. Waits for the call, then writes the summed
 * milliseconds of each phase class to class_ms_h: 0 the RMSNorms (and the first layer's embedding gather), 1 the
 * projections q|k|v, o, gate|up and down (GEMMs and their epilogues), 2 attention (K/V write, chunk attention,
 * merge), 3 the output head and its argmax. Codes: 578 (class_ms_h NULL), 577 (len_class_ms < 4), then as
 * llmk_prefill. On success slot_len_h[slot] = pos0 + n. */
int32_t llmk_prefill_profiled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                              const int64_t* tokens_h, int64_t n, int64_t pos0, int32_t* tokens_out,
                              int64_t len_tokens, float* class_ms_h, int64_t len_class_ms, void* ws, int64_t len_ws,
                              void* stream);

/* ------------------------------------------------------------------------- */
/* int8 weight packs (LLMK_Q8)                                                */
/* ------------------------------------------------------------------------- */
/* Decode reads packed int8 weights in [xpu] "1. CausalLM: the forward path" (and an int8 GPU kernel stands
 * beside the CPU reference in [llmk] "How this composes into a decode step"), with no layout given; this
 * format is the library's own. A q8 pack holds a rows x cols matrix, output-major (each row is one
 * output's weights over cols inputs), in groups of LLMK_Q8_GROUP consecutive inputs of a row: per group the
 * fp32 scale s = max|w| / 127 and int8 codes q = rint(w / s) (ties to even; 0 for an all-zero group),
 * decided in fp32; the weight is q * s, |w - q s| <= s / 2. Bytes: rows*cols codes row-major, then
 * rows*(cols/LLMK_Q8_GROUP) fp32 scales row-major: 1 + 4/128 bytes a weight against 2 for bf16.
 * A model with w_dtype LLMK_Q8 holds q8 packs, in LLMK_W_OUT_IN, for wq [H*hd x d], wk, wv [Hkv*hd x d],
 * wo [d x H*hd], w_gate, w_up [F x d], w_down [d x F] and w_out [vocab x d] (each llmk_tensor.len is the
 * pack's byte count, the pointer 16-byte aligned) and the embedding table in bf16 (vocab*d elements).
 * d, H*hd and F are multiples of LLMK_Q8_GROUP, at most 16,384. Such a model runs llmk_decode_step,
 * llmk_decode_steps (sampled too) and the timing aids, in the persistent form where it can run (head_dim
 * 64..256, a bf16 or fp32 K/V cache) and else one kernel per operation; the batched step and prefill refuse
 * it (578). */
#define LLMK_Q8_GROUP 128

/* Bytes of a q8 pack of a rows x cols matrix, or -1 if rows or cols is < 1 or > LLMK_MAX_DIM or cols is not
 * a multiple of LLMK_Q8_GROUP. */
int64_t llmk_q8_pack_bytes(int64_t rows, int64_t cols);

/* Quantize w (device, rows x cols row-major, output-major, w_dtype LLMK_F32 or LLMK_BF16, finite values)
 * into the q8 pack at `pack` (device, len_pack bytes), on `stream`. Both w and pack must be 16-byte aligned
 * (the decode step reads packs with 16-byte loads). Codes: 578 (null, w_dtype), 561 (rows or cols < 1),
 * 564 (> LLMK_MAX_DIM), 574 (cols not a multiple of LLMK_Q8_GROUP), 576 (len_w != rows*cols), 577 (len_pack
 * != llmk_q8_pack_bytes), 578 (w or pack not 16-byte aligned), 579 (launch failed). */
int32_t llmk_quantize_q8(const void* w, int64_t len_w, int32_t w_dtype, int64_t rows, int64_t cols, void* pack,
                         int64_t len_pack, void* stream);

/* dst = src^T for a rows x cols row-major matrix (dst is cols x rows), both device buffers of rows*cols
 * elements of dtype; the one-time repacking of projections into LLMK_W_OUT_IN. dst may not alias src.
 * Codes: 578 (null, dtype, aliasing), 561, 564, 562 (len_src), 577 (len_dst). */
int32_t llmk_transpose(const void* src, int64_t len_src, void* dst, int64_t len_dst, int64_t rows, int64_t cols,
                       int32_t dtype, void* stream);

/* Measurement aid (not on the decode path): the number of kernels one decode step launches, in launch
 * order per layer q|k|v, attention, o, gate|up, down, then the output head (5 * n_layer + 1), or a
 * negative status if cfg is refused. */
int64_t llmk_decode_kernel_count(const llmk_config* cfg);

/* One decode step exactly as llmk_decode_step (logits and hidden not returned), with a HIP event
 * recorded on `stream` right before and right after every kernel launch. Waits for the step, then
 * writes each kernel's duration in milliseconds to kernel_ms_h[k] (host, len_kernel_ms >=
 * llmk_decode_kernel_count(cfg)), in launch order. Codes: as llmk_decode_step; 578 if kernel_ms_h is
 * NULL; 577 if len_kernel_ms is too small. On success slot_len_h[slot] becomes pos + 1. */
int32_t llmk_decode_step_profiled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                  int64_t token, int64_t pos, int32_t* token_out, float* kernel_ms_h,
                                  int64_t len_kernel_ms, void* ws, int64_t len_ws, void* stream);

/* Which form llmk_decode_step / llmk_decode_steps take for this config on the current device:
 * LLMK_STEP_PER_OP or LLMK_STEP_PERSISTENT (AUTO resolved). Host-side; queries the device.
 * Codes: the config's check code if it is invalid; 578 if the config asks for LLMK_STEP_PERSISTENT where it
 * cannot run. */
int32_t llmk_decode_path(const llmk_config* cfg);

/* Measurement aid (not on the decode path): the average duration of one launch of one of the step's
 * kernel classes, timed the way the step runs it. kernel: 0 q|k|v, 1 attention, 2 o, 3 gate|up, 4 down,
 * 5 output head (the kernels of the per-operation form), 6 the persistent step kernel (the whole step;
 * 578 where the config does not run it). For 6 the `reps` launches are `reps` consecutive steps from
 * (token, pos) replayed as one captured launch; they also write K/V rows at positions pos + 1 ..
 * pos + reps - 1, past the slot's length (571 if pos + reps exceeds the capacity). Runs one ordinary decode step at (token, pos), captures that class's launches for every
 * layer (the head: once), `reps` times over, back to back into one HIP graph, replays it once between two
 * HIP events recorded on `stream`, then runs the ordinary step at (token, pos) once more. The repeated
 * launches work on the workspace only (the head's tokens go to workspace scratch, never to token_out), and
 * the final step rewrites what they disturbed, so the call leaves the pool, token_out (the greedy token)
 * and slot_len_h[slot] = pos + 1 exactly as llmk_decode_step does. *ms_per_launch_h (host) receives the
 * elapsed time divided by the number of launches. Synchronizes `stream`.
 * Codes: as llmk_decode_step; 578 if ms_per_launch_h is NULL or kernel is not 0..6; 561 if reps < 1; 564
 * if reps > 64. */
int32_t llmk_decode_kernel_time(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                int64_t token, int64_t pos, int32_t kernel, int32_t reps, int32_t* token_out,
                                float* ms_per_launch_h, void* ws, int64_t len_ws, void* stream);

/* Measurement aid for the batched step, as llmk_decode_kernel_time: the average duration of one launch of
 * one kernel class of llmk_decode_step_batch. kernel: 0 attention-side RMSNorm, 1 q|k|v, 2 attention,
 * 3 o, 4 FFN-side RMSNorm, 5 gate|up, 6 down, 7 final RMSNorm, 8 output head with argmax. Runs one
 * ordinary batched step, replays that class's launches (every layer; the last two once) `reps` times in
 * one graph between two HIP events on `stream`, then runs the ordinary step once more, so the call leaves
 * the pool, tokens_out and every slot length exactly as llmk_decode_step_batch does (tokens_out: device
 * int32 [batch]). Codes: as llmk_decode_step_batch; 578 if ms_per_launch_h is NULL or kernel is not 0..8;
 * 561 if reps < 1; 564 if reps > 64. */
int32_t llmk_decode_batch_kernel_time(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool,
                                      int64_t batch, const int64_t* slots_h, const int64_t* tokens_h,
                                      const int64_t* pos_h, int32_t kernel, int32_t reps, int32_t* tokens_out,
                                      float* ms_per_launch_h, void* ws, int64_t len_ws, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLMK_H */
