// Launch interface of the gfx950 kernels (host side of libllmk).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace llmk {

// ------------------------------------------------------------------------------------------------
// Transposed GEMV, y = A^T x, split over K with a deterministic last-block reduction.
// ------------------------------------------------------------------------------------------------

enum GemvMode { GM_PLAIN = 0, GM_QKV = 1, GM_RESID = 2, GM_GATEUP = 3 };

struct GemvParams {
  // weights ([in][out] row-major). PLAIN/RESID: w0. GATEUP: w0 = gate, w1 = up (same shape).
  // QKV: w0 = wq (n0 columns), w1 = wk (n1 columns), w2 = wv (N - n0 - n1 columns).
  const void* w0;
  const void* w1;
  const void* w2;
  int64_t n0, n1;
  int64_t K, N;            // rows of A (= length of the input), output columns
  int64_t rows_per_split;  // rows handled by one workgroup
  int32_t ksplit, n_cblk;  // grid = ksplit * n_cblk workgroups
  int32_t lpr;             // lanes per row segment (16, 32 or 64): a workgroup owns lpr * VEC columns
  // input vector of length K: fp32, or a row of the weight dtype (the embedding table) chosen by token
  const void* in;
  int32_t in_is_w;               // 1: `in` has the weight dtype
  const DecodeState* in_state;   // non-null: in += state->token * K (embedding row)
  const float* gain;             // non-null: RMSNorm the input first (h = in * rsqrt(mean(in^2)+eps) * gain)
  float eps;
  // split-K workspace
  float* partial;                // [ksplit][NACC][N]
  unsigned* counters;            // [n_cblk], zero on entry, left zero on exit
  // epilogue
  float* y;                      // PLAIN and QKV: y[N] (q|k|v raw); GATEUP: u[N]
  float* x;                      // RESID: residual stream, x = base + A^T in
  const void* base;              // RESID: base (fp32 x itself, or the embedding table of weight dtype)
  int32_t base_is_w;             // 1: base is the embedding table, row chosen by base_state->token
  const DecodeState* base_state;
  float* hidden;                 // RESID: optional copy of the new x
};

// Fills lpr/ksplit/n_cblk/rows_per_split for a K x N problem: about target_blocks workgroups, each
// owning at least min_cols output columns (the q|k|v epilogue needs whole heads in one workgroup).
void gemv_plan(GemvParams& p, int w_is_bf16, int vec1, int target_blocks, int min_cols);
hipError_t gemv_launch(const GemvParams& p, int mode, int w_is_bf16, int vec1, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Untransposed GEMV (row dots), the output head: y[r] = W[r] . h, optionally h = rmsnorm(x) * gain,
// optionally followed by the greedy argmax of y.
// ------------------------------------------------------------------------------------------------

struct HeadParams {
  const void* w;          // [rows][cols]
  int64_t rows, cols;
  int64_t rows_per_block;
  int32_t n_blocks;
  const float* x;         // [cols]
  const float* gain;      // non-null: RMSNorm first
  float eps;
  float* y;               // [rows]
  // argmax (when part_val != nullptr)
  float* part_val;        // [n_blocks]
  int32_t* part_idx;      // [n_blocks]
  unsigned* counter;      // one counter, zero on entry and exit
  int32_t* token_out;     // token written at token_out[state ? state->step : 0]
  float* logit_out;       // optional
  DecodeState* state;     // optional: token <- argmax, pos += 1, step += 1
};

void head_plan(HeadParams& p, int w_is_bf16);
hipError_t head_launch(const HeadParams& p, int w_is_bf16, hipStream_t s);
hipError_t rowdot_simple_launch(const void* w, int w_is_bf16, const float* x, float* y, int64_t rows, int64_t cols,
                                hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Row-dot GEMV over output-major weights (W [rows][K]): y[r] = W[r] . h with per-row epilogues.
// ------------------------------------------------------------------------------------------------

constexpr int RD_MAX_ROWS = 256;   // rows one workgroup owns, at most

struct RowdotParams {
  const void* w0;          // PLAIN/RESID: the matrix; GATEUP: gate; QKV: wq
  const void* w1;          // GATEUP: up; QKV: wk
  const void* w2;          // QKV: wv
  int64_t n0, n1;          // QKV: rows of wq and wk
  int64_t N, K;            // output rows, input length
  int64_t rows_per_block;
  int32_t n_blocks, kw, np, r;
  const void* in;          // input: fp32, or the embedding row (weight dtype) chosen by in_state->token
  int32_t in_is_w;
  const DecodeState* in_state;
  const float* gain;       // non-null: RMSNorm the input first
  float eps;
  float* y;                // PLAIN/QKV: y[N]; GATEUP: u[N]
  float* x;                // RESID: x = base + y
  const void* base;
  int32_t base_is_w;
  const DecodeState* base_state;
  float* hidden;
};

// Fills kw/np/r/rows_per_block/n_blocks (N and K set); -1 if K does not fit the kernel.
int rowdot_plan(RowdotParams& p, int w_is_bf16, int mode);
hipError_t rowdot_launch(const RowdotParams& p, int mode, int w_is_bf16, hipStream_t s);
hipError_t transpose_launch(const void* src, void* dst, int64_t rows, int64_t cols, int is_bf16, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Batched projections on matrix cores: Y[b][n] = W[n] . X[b] for up to 64 rows b, W bf16 output-major,
// X given as bf16 hi and lo parts ([64][K] each, row stride K).
// ------------------------------------------------------------------------------------------------

// Prefill projections: Y = X W^T over a chunk of M rows, 128 x 128 tiles, K split where the tiles alone do
// not fill the chip; the epilogue adds the splits in order and applies the operation.
enum PgemmMode { PG_NONE = 0, PG_STORE = 1, PG_RESID = 2, PG_GATEUP = 3 };
struct PgemmParams {
  const bf16_t* ahi;      // X as bf16 hi + lo, [M][lda]
  const bf16_t* alo;
  int64_t lda;
  const void* w0;         // W rows (bf16, K each): [0, n0) of w0, then n1 rows of w1, then the rest of w2
  const void* w1;
  const void* w2;
  int64_t n0, n1;
  int32_t M;
  int32_t ksplit;
  int64_t N, K;
  int64_t kslice;         // k per split (a multiple of 32)
  float* y;               // [ksplit][M][N] partial tiles (PG_NONE with one split: the result itself)
  float* out;             // PG_STORE: out[m * ldo + n] = y; PG_RESID: out[m * ldo + n] += y
  int64_t ldo;
  float* hidden;          // PG_RESID, optional: hidden[m * hidden_stride + n] = the updated out
  int64_t hidden_stride;
  bf16_t* uhi;            // PG_GATEUP: silu(gate) * up as hi + lo, [M][N / 2] (gate rows first, then up)
  bf16_t* ulo;
};
void pgemm_plan(PgemmParams& p, int target_blocks);
hipError_t pgemm_launch(const PgemmParams& p, int mode, hipStream_t s);

// Prefill attention: 64 query vectors of one K/V head (chunk rows x its query heads) per workgroup over one
// part of FA_SPAN positions, then a merge of the parts per (row, head) into the output as hi + lo.
constexpr int FA_SPAN = 256;
struct FattnParams {
  const float* qkv;            // [rows][qkv_stride] raw q|k|v (q unrotated)
  int64_t qkv_stride;
  const BatchState* st;        // row r: position pos[r], slot slot[r] (one slot for the chunk)
  int32_t rows;
  int32_t H, Hkv;
  const void* k;               // this layer's K / V pool buffers, the chunk's rows already appended
  const void* v;
  int32_t kv_is_bf16;
  int64_t slot_elems;
  KvPaging pg;                 // paged pool: rows through the chunk slot's table row (then slot_elems unused)
  const float* rope_table;
  int32_t rope_layout;
  int32_t span;                // FA_SPAN
  int32_t n_parts;             // capacity of `part` in parts per (row, head)
  float* part;                 // [rows][H][n_parts][hd + 2]: unnormalised output, max, sum
  bf16_t* out_hi;              // [rows][H * hd]
  bf16_t* out_lo;
};
// the chunk attention takes head dim 128, at most 64 query heads per K/V head and contexts up to 8,192 positions
bool fattn_supported(int64_t H, int64_t Hkv, int64_t hd, int64_t max_ctx);
int64_t fattn_parts(int64_t max_ctx);
hipError_t fattn_launch(const FattnParams& p, int64_t max_ctx, hipStream_t s);

// h[b] = rmsnorm(x[b]) * gain split into hi/lo, for rows b < rows; with emb, x[b] is first set to the
// embedding row of state->token[b] (the first layer).
hipError_t bnorm_launch(float* x, const void* emb, int emb_is_bf16, const BatchState* state, int32_t rows, int64_t d,
                        const float* gain, float eps, bf16_t* hhi, bf16_t* hlo, hipStream_t s);
struct BatchInit {
  int32_t token[LLMK_MAX_BATCH_ROWS];
  int32_t pos[LLMK_MAX_BATCH_ROWS];
  int32_t slot[LLMK_MAX_BATCH_ROWS];
  int32_t rows;
};
hipError_t set_batch_state_launch(BatchState* st, const BatchInit& init, hipStream_t s);
// After the batched head: row b's greedy token tok[b] goes to token_out[step * rows + b] and becomes the row's
// next input, its position advances, and the step count too.
hipError_t batch_advance_launch(BatchState* st, const int32_t* tok, int32_t* token_out, int32_t rows, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Split-context grouped-query attention for one query position, plus the log-sum-exp merge.
// ------------------------------------------------------------------------------------------------

struct AttnParams {
  const float* q;        // [H][hd]
  const void* k;         // [>= ctx][Hkv][hd] (the sequence's region)
  const void* v;
  int32_t kv_is_bf16;
  int32_t kv_q8;               // int8 cache: k / v hold codes, k_scale / v_scale one scale per (row, K/V head)
  const float* k_scale;        // [rows][Hkv], rows counted as for k (the slot's region, or the block store)
  const float* v_scale;
  float* k_scale_w;
  float* v_scale_w;
  int32_t H, Hkv, hd;
  int32_t ctx;                 // used when state == nullptr
  const DecodeState* state;    // non-null: ctx = state->pos + 1
  int32_t chunk;               // positions per sub-chunk (<= 64)
  int32_t sub_per_wg;          // consecutive sub-chunks one workgroup walks (online softmax)
  int32_t n_parts;             // grid.x; parts past ctx exit at once (<= ATTN_MAX_PARTS)
  float* part;                 // [Hkv][n_parts][G][hd + 2]: max, sum, unnormalised output
  unsigned* counters;          // [Hkv], zero on entry and exit
  float* out;                  // [H][hd]
  // decode step: q|k|v of this position arrive unrotated; q and k are rotated by the position here and
  // k, v are appended (rounded to the cache dtype) to k_w / v_w, the writable views of k / v
  const float* qkv_raw;        // [H*hd | Hkv*hd | Hkv*hd] or nullptr (then q is used as given)
  void* k_w;
  void* v_w;
  const float* rope_table;     // [max_pos][hd/2][2]
  int32_t rope_layout;
  int32_t no_append;           // prefill: k, v of every row are already in the cache; rotate q only
  // batched decode (bstate non-null): grid.z = rows; row r reads pos and slot from bstate, its K/V region
  // starts slot * slot_elems elements into k / v / k_w / v_w, its q|k|v at qkv_raw + r * qkv_stride, and
  // its output goes, split into bf16 hi/lo, to out_hi / out_lo + r * H * hd
  const BatchState* bstate;
  int32_t rows;                // grid.z when bstate is set
  int64_t slot_elems;
  // paged pool (pg.table set): position t of the sequence is cache row kv_block_row(trow, pg.shift, t) of
  // k / v / k_w / v_w (no slot offset), trow = pg.table (single sequence: its own row) or, batched,
  // pg.table + slot * pg.stride
  KvPaging pg;
  int64_t qkv_stride;
  bf16_t* out_hi;
  bf16_t* out_lo;
  // persistent decode step (tagged form): q|k|v and the output as tagged activations (act_tag in the two
  // low mantissa bits, see attn_block), the parts as (value, part_tag) pairs
  const uint32_t* qkv_tag;
  uint32_t* out_tag;
  uint32_t tag;                // the activations' tag of this step (1 or 2; 3, which no step writes: give-up tests)
  uint32_t part_tag;           // the parts' tag: unique per (step, layer), the part buffer serves every layer
  uint64_t* part_tagged;       // [Hkv][n_parts][G][hd + 2] (value, part_tag) pairs
  int32_t* err;
};

constexpr int ATTN_MAX_PARTS = 32;
// Fills chunk / sub_per_wg / n_parts for contexts up to max_ctx.
// min_tiles_per_part: the fewest tiles one part should take (parts are capped at ATTN_MAX_PARTS either way).
void attn_plan(AttnParams& p, int64_t max_ctx, int64_t min_tiles_per_part = 1);
hipError_t attn_launch(const AttnParams& p, hipStream_t s);
inline int64_t attn_part_floats(int64_t H, int64_t hd) { return (int64_t)ATTN_MAX_PARTS * H * (hd + 2); }

// ------------------------------------------------------------------------------------------------
// The persistent decode-step kernel (one launch per step, one workgroup per CU)
// ------------------------------------------------------------------------------------------------

struct StepLayer {
  const bf16_t* w[7];      // wq, wk, wv, wo, gate, up, down, output-major
  const float* g1;         // attention-side RMSNorm gain
  const float* g2;         // FFN-side RMSNorm gain
  void* k;                 // this layer's K and V pool buffers (slot 0)
  void* v;
};

struct StepParams {
  const StepLayer* layers;      // device table [n_layer]
  const bf16_t* emb;
  const bf16_t* w_out;
  const float* g_final;
  const float* rope_table;
  int32_t n_layer, d, qd, kvd, F, V, H, Hkv, hd, rope_layout;
  float eps;
  int32_t nwg;                  // workgroups (one per CU)
  int64_t kv_off;               // element offset of the slot in each pool buffer (0 for a paged pool)
  const int32_t* kv_table;      // paged pool: the slot's row of the block table (else nullptr)
  int32_t kv_shift;             // log2 of the positions per block
  int32_t attn_chunk;           // positions per attention tile
  int32_t give_up;              // test only: the attention waits for a tag nobody writes (bounded-wait path)
  int32_t qw;                   // the projections and the head are int8 packs (layers' w[] and w_out point at packs)
  DecodeState* state;
  // activations as tagged fp32 words (act_tag(step) in the two low mantissa bits); cleared before each call.
  // x [2 n_layer][x_stride]: x after layer l's o (2l) and after its down (2l + 1); q|k|v, attention
  // output and u [n_layer][*_stride]
  uint32_t* x;
  uint32_t* qkv;
  uint32_t* att;
  uint32_t* u;
  int64_t x_stride, qkv_stride, att_stride, u_stride;
  uint64_t* attn_part;          // [Hkv][ATTN_MAX_PARTS][G][hd + 2] (value, tag) pairs, tag unique per layer
  float* logits;                // optional [V]
  float* hidden;                // optional [n_layer][d]
  float* head_val;              // [nwg]
  int32_t* head_idx;
  unsigned* head_cnt;           // zero on entry and exit
  int32_t* err;                 // set when a wait gives up
  int32_t* token_out;           // token of step s at token_out[s]
};

constexpr int STEP_MAX_LAYERS = 128;   // layers the persistent step kernel supports
constexpr int STEP_MAX_VIN = 16384;    // longest projection input (d, H*hd, hidden) it supports
constexpr int STEP_MAX_RES = 256;      // residual rows per workgroup (d / workgroups, rounded up) it supports
constexpr int STEP_MAX_WAVE_ROWS = 128;  // output rows one wave of it holds (gate|up: gate and up rows count apart)
// Workgroups the step kernel runs with on the current device (0 if it cannot hold one per CU); qw: int8 packs.
int step_grid(int kv_is_bf16, int hd, int qw);
hipError_t step_launch(const StepParams& p, int kv_is_bf16, hipStream_t s);
struct StepTableChunk {
  StepLayer layers[8];
  int32_t first, count;
};
hipError_t step_table_launch(StepLayer* dst, const StepTableChunk& chunk, hipStream_t s);

// ------------------------------------------------------------------------------------------------
// Elementwise and small kernels
// ------------------------------------------------------------------------------------------------

hipError_t residual_add_launch(const float* a, const float* b, float* out, int64_t n, hipStream_t s);
hipError_t add_rmsnorm_launch(float* residual, const float* x, const float* gain, int64_t rows, int64_t n, float eps,
                              float* h, hipStream_t s);
hipError_t silu_mul_launch(const float* gate, const float* up, float* out, int64_t n, hipStream_t s);
hipError_t rope_table_launch(float* table, int64_t max_pos, int64_t hd, double base, hipStream_t s);
hipError_t rope_launch(float* q, float* k, int64_t rows, int64_t nq, int64_t nk, int64_t hd, const int32_t* pos,
                       int64_t max_pos, const float* table, int layout, hipStream_t s);
hipError_t kv_append_launch(void* cache, int is_bf16, int64_t offset, const float* src, int64_t n, hipStream_t s);
// Paged append: element f = first + i (i < n) of a slot's flat cache goes to position f / row_elems, element
// f % row_elems, through the slot's table row trow (blocks of 1 << shift positions).
hipError_t kv_append_paged_launch(void* cache, int is_bf16, const int32_t* trow, int shift, int64_t row_elems,
                                  int64_t first, const float* src, int64_t n, hipStream_t s);
// Block-table writes: table[idx[i]] = val[i] for i < n, carried by value in the launch.
constexpr int TABLE_EDITS = 48;
struct TableEdits {
  int64_t idx[TABLE_EDITS];
  int32_t val[TABLE_EDITS];
  int32_t n;
};
hipError_t table_set_launch(int32_t* table, const TableEdits& e, hipStream_t s);
constexpr int SAMPLE_MAX_K = 1024;   // survivors (top-k after clamping to the row length) the sampler holds
enum SampleForm { SAMPLE_WIDE = 0, SAMPLE_WAVE_SLICES = 1, SAMPLE_BLOCK_SLICES = 2 };
struct SamplePlan {
  int form;        // SampleForm
  int slices;      // per row (1 for the wide form)
  int64_t chunk;   // logits per slice
};
SamplePlan sample_plan(int64_t n, int32_t k);
int64_t sample_workspace_bytes(int64_t rows, int64_t n, int32_t k);
hipError_t sample_launch(const float* logits, int64_t rows, int64_t n, float temperature, int32_t k, float top_p,
                         const float* draw, int32_t* token, void* ws, hipStream_t s);
hipError_t argmax_launch(const float* logits, int64_t rows, int64_t n, int32_t* token, float* logit, float* part_val,
                         int32_t* part_idx, unsigned* counters, int32_t blocks_per_row, hipStream_t s);
hipError_t fill_u32_launch(unsigned* p, int64_t n, unsigned v, hipStream_t s);
// Prefill: for every row r of the batch state, rotate its k by pos[r], round k and v to the cache dtype and
// store them at pos[r] of slot[r] (k, v: one layer's pool buffers; qkv: [rows][qkv_stride] raw q|k|v).
// kv_dtype LLMK_Q8: each (row, K/V head) of k and v is quantized to codes and a scale (k_scale, v_scale: the
// buffers' scales, one per cache row and K/V head).
hipError_t rope_append_rows_launch(const float* qkv, int64_t qkv_stride, const BatchState* st, int32_t rows,
                                   int32_t H, int32_t Hkv, int32_t hd, const float* rope_table, int32_t rope_layout,
                                   void* k, void* v, int32_t kv_dtype, int64_t slot_elems, const KvPaging& pg,
                                   float* k_scale, float* v_scale, hipStream_t s);
hipError_t set_state_launch(DecodeState* st, int32_t token, int32_t pos, hipStream_t s);

}  // namespace llmk
