// C ABI of libllmk: host-side checks (all before any HIP call), workspace layout and the assembly of
// the decode step from the gfx950 kernels. See include/llmk.h for the contract of every entry point.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <string.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "kvpages.h"
#include "loop.h"
#include "q8.h"
#include "llmk.h"

using namespace llmk;

// Scratch of llmk_argmax_noalloc, for callers that cannot allocate: the per-block partials and tickets of
// LLMK_ARGMAX_NOALLOC_MAX_ROWS rows of at most 64 blocks each (two 64 KiB partial arrays and the tickets,
// each region 256-byte aligned). Every GPU the library runs this entry point on holds its own copy until
// the process ends. Host code never uses this name as an address: it asks the runtime for the array's
// address on each device once and passes that pointer.
static constexpr int64_t kArgmaxScratchBytes = 2 * 65536 + 1024;
static __device__ __align__(256) unsigned char scratch[kArgmaxScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device `stream` runs on, looked up once per device with that device
// current (nullptr on failure).
void* scratch_on(hipStream_t stream) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  hipDevice_t dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

constexpr int64_t kMaxDim = LLMK_MAX_DIM;
constexpr int64_t kAlign = 256;

inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// 561 / 564 over a list of dimensions (all must be >= 1)
int32_t dims_check(std::initializer_list<int64_t> dims) {
  for (int64_t d : dims)
    if (d < 1) return LLMK_EMPTY_DIMENSION;
  for (int64_t d : dims)
    if (d > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  return LLMK_OK;
}

inline bool is_dtype(int32_t t) { return t == LLMK_F32 || t == LLMK_BF16; }
inline bool is_kv_dtype(int32_t t) { return is_dtype(t) || t == LLMK_Q8; }
inline int64_t dtype_size(int32_t t) { return t == LLMK_Q8 ? 1 : t == LLMK_BF16 ? 2 : 4; }
inline bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline bool rope_head_dim_ok(int64_t hd) { return hd >= 2 && hd <= 256 && hd % 2 == 0; }
inline bool attn_head_dim_ok(int64_t hd) { return hd >= 2 && hd <= 256 && pow2(hd); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t finish(hipError_t e) { return e == hipSuccess ? LLMK_OK : LLMK_DEVICE_ERROR; }

// Workspace carving: a bump allocator over the caller's buffer (nullptr base = size query).
struct Carve {
  char* base;
  int64_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T> T* take(int64_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * (int64_t)sizeof(T));
    return p;
  }
};

// ---- gemv_t plan shared by the primitive and its workspace query ---------------------------------------

struct GemvT {
  GemvParams p{};
  int vec1 = 0;
};

GemvT plan_gemv_t(int64_t m, int64_t n, int32_t dt, const void* a) {
  GemvT g;
  const int64_t vec = dt == LLMK_BF16 ? 8 : 4;
  g.vec1 = (n % vec != 0) || (a && !aligned16(a));
  g.p.K = m;
  g.p.N = n;
  gemv_plan(g.p, dt == LLMK_BF16, g.vec1, 512, 0);
  return g;
}

int64_t gemv_t_ws(const GemvT& g) {
  if (g.p.ksplit <= 1) return 0;
  Carve c(nullptr);
  c.take<float>((int64_t)g.p.ksplit * g.p.N);
  c.take<unsigned>(g.p.n_cblk);
  return c.off;
}

// Workspace for either path (vector or scalar), so the answer does not depend on the pointer's alignment.
int64_t gemv_t_ws_any(int64_t m, int64_t n, int32_t dt) {
  int64_t w = gemv_t_ws(plan_gemv_t(m, n, dt, nullptr));
  GemvT s;
  s.vec1 = 1;
  s.p.K = m;
  s.p.N = n;
  gemv_plan(s.p, dt == LLMK_BF16, 1, 512, 0);
  const int64_t ws = gemv_t_ws(s);
  return ws > w ? ws : w;
}

// ---- decode plan --------------------------------------------------------------------------------------

int32_t config_check(const llmk_config* c) {
  if (!c) return LLMK_INVALID_ARGUMENT;
  if ((!is_dtype(c->w_dtype) && c->w_dtype != LLMK_Q8) || !is_kv_dtype(c->kv_dtype)) return LLMK_INVALID_ARGUMENT;
  if (c->rope_layout != LLMK_ROPE_HALF_SPLIT && c->rope_layout != LLMK_ROPE_INTERLEAVED) return LLMK_INVALID_ARGUMENT;
  if (c->w_layout != LLMK_W_IN_OUT && c->w_layout != LLMK_W_OUT_IN) return LLMK_INVALID_ARGUMENT;
  if (c->step_path != LLMK_STEP_AUTO && c->step_path != LLMK_STEP_PER_OP && c->step_path != LLMK_STEP_PERSISTENT)
    return LLMK_INVALID_ARGUMENT;
  if (c->test_flags != 0 && c->test_flags != LLMK_TEST_WAIT_GIVE_UP) return LLMK_INVALID_ARGUMENT;
  if (!(c->eps > 0) || !isfinite(c->eps) || !(c->rope_base > 1.0) || !isfinite(c->rope_base))
    return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({c->vocab, c->d, c->n_layer, c->n_head, c->n_kv, c->head_dim, c->hidden, c->max_seq});
  if (st != LLMK_OK) return st;
  if (c->n_head % c->n_kv != 0 || c->n_head / c->n_kv > 8 || !attn_head_dim_ok(c->head_dim))
    return LLMK_HEAD_SHAPE_INVALID;
  if (c->kv_dtype == LLMK_Q8 && c->head_dim % 16 != 0) return LLMK_HEAD_SHAPE_INVALID;   // whole 16-code loads
  if (c->kv_dtype == LLMK_Q8 && c->step_path == LLMK_STEP_PERSISTENT) return LLMK_INVALID_ARGUMENT;
  if (c->w_dtype == LLMK_Q8) {
    // int8 packs: the inputs of every projection and of the head in whole groups, a row segment per lane
    const int64_t ks[3] = {c->d, c->n_head * c->head_dim, c->hidden};
    for (int64_t k : ks) {
      RowdotParams r{};
      r.K = k;
      r.N = 1;
      if (rowdot_q8_plan(r, GM_PLAIN) != 0) return LLMK_HEAD_SHAPE_INVALID;
    }
    if (c->w_layout != LLMK_W_OUT_IN) return LLMK_INVALID_ARGUMENT;
    return LLMK_OK;
  }
  const int64_t vec = c->w_dtype == LLMK_BF16 ? 8 : 4;
  const int64_t widths[4] = {c->d, c->n_head * c->head_dim, c->n_kv * c->head_dim, c->hidden};
  for (int64_t w : widths)
    if (w % vec != 0) return LLMK_HEAD_SHAPE_INVALID;
  if (c->d > 64 * vec * 16) return LLMK_HEAD_SHAPE_INVALID;  // the head kernel holds d in registers
  if (c->w_layout == LLMK_W_OUT_IN) {   // the row-dot kernels hold a K segment per lane in registers
    const int64_t ks[3] = {c->d, c->n_head * c->head_dim, c->hidden};
    for (int64_t k : ks) {
      RowdotParams r{};
      r.K = k;
      r.N = 1;
      if (rowdot_plan(r, c->w_dtype == LLMK_BF16, GM_PLAIN) != 0) return LLMK_HEAD_SHAPE_INVALID;
    }
  }
  if (c->step_path == LLMK_STEP_PERSISTENT && (c->w_dtype != LLMK_BF16 || c->w_layout != LLMK_W_OUT_IN))
    return LLMK_INVALID_ARGUMENT;
  return LLMK_OK;
}

struct DecodePlan {
  int rowdot = 0;                       // 1: output-major weights (row-dot kernels), 0: split-K kernels
  GemvParams qkv{}, o{}, gu{}, down{};
  RowdotParams rqkv{}, ro{}, rgu{}, rdown{};
  int q8 = 0;                           // 1: int8 weight packs (row-dot over packs, head as row-dot + argmax)
  RowdotParams rhead{};
  int32_t* q8_tok = nullptr;            // the int8 head's greedy token
  float* draw1 = nullptr;               // the sampled loop: this step's uniform
  int32_t* sampled_tok = nullptr;       // and its token
  HeadParams head{};
  AttnParams attn{};
  // workspace regions
  DecodeState* state = nullptr;
  float* x = nullptr;
  float* qkv_buf = nullptr;             // raw q|k|v of the step's position
  float* att = nullptr;
  float* u = nullptr;
  float* logits = nullptr;
  float* partial = nullptr;
  unsigned* counters = nullptr;
  float* attn_part = nullptr;
  float* head_val = nullptr;
  int32_t* head_idx = nullptr;
  int32_t* tok_scratch = nullptr;   // kTimeMaxReps tokens: where repeated timing launches of the head write
  // persistent step
  StepLayer* step_layers = nullptr;     // [n_layer]
  int32_t* step_err = nullptr;          // error flag, zero per call
  unsigned* step_cnt = nullptr;         // the head's ticket
  float* step_val = nullptr;            // [kStepMaxWG] per-workgroup best logit
  int32_t* step_idx = nullptr;
  uint32_t* step_tagged = nullptr;      // the tagged activations and parts below, one region cleared per call
  int64_t step_tagged_words = 0;        // its 4-byte words
  uint32_t* step_x = nullptr;           // tagged activations of the persistent step (see StepParams)
  uint32_t* step_qkv = nullptr;
  uint32_t* step_att = nullptr;
  uint32_t* step_u = nullptr;
  uint64_t* step_part = nullptr;        // attention parts as (value, tag) pairs
  int64_t step_x_stride = 0, step_qkv_stride = 0, step_att_stride = 0, step_u_stride = 0;
  int64_t bytes = 0;
  int n_gemv_counters = 0;
};

constexpr int kGemvTargetBlocks = 512;
constexpr int kTimeMaxReps = 64;   // llmk_decode_kernel_time: at most this many replays of a kernel class
constexpr int kStepMaxWG = 1024;   // the persistent step kernel's workgroups (one per CU), at most


void plan_decode(const llmk_config* c, void* ws, DecodePlan& D) {
  const int bf = c->w_dtype == LLMK_BF16;
  const int64_t d = c->d, qd = c->n_head * c->head_dim, kvd = c->n_kv * c->head_dim, F = c->hidden;
  D.qkv.K = d; D.qkv.N = qd + 2 * kvd; D.qkv.n0 = qd; D.qkv.n1 = kvd;
  D.o.K = qd; D.o.N = d;
  D.gu.K = d; D.gu.N = F;
  D.down.K = F; D.down.N = d;
  gemv_plan(D.qkv, bf, 0, kGemvTargetBlocks, 0);
  gemv_plan(D.o, bf, 0, kGemvTargetBlocks, 0);
  gemv_plan(D.gu, bf, 0, kGemvTargetBlocks, 0);
  gemv_plan(D.down, bf, 0, kGemvTargetBlocks, 0);
  D.rowdot = c->w_layout == LLMK_W_OUT_IN;
  D.rqkv.K = d; D.rqkv.N = qd + 2 * kvd; D.rqkv.n0 = qd; D.rqkv.n1 = kvd;
  D.ro.K = qd; D.ro.N = d;
  D.rgu.K = d; D.rgu.N = F;
  D.rdown.K = F; D.rdown.N = d;
  D.q8 = c->w_dtype == LLMK_Q8;
  if (D.q8) {
    D.rhead.K = d; D.rhead.N = c->vocab;
    rowdot_q8_plan(D.rqkv, GM_QKV);
    rowdot_q8_plan(D.ro, GM_RESID);
    rowdot_q8_plan(D.rgu, GM_GATEUP);
    rowdot_q8_plan(D.rdown, GM_RESID);
    rowdot_q8_plan(D.rhead, GM_PLAIN);
  } else if (D.rowdot) {
    rowdot_plan(D.rqkv, bf, GM_QKV);
    rowdot_plan(D.ro, bf, GM_RESID);
    rowdot_plan(D.rgu, bf, GM_GATEUP);
    rowdot_plan(D.rdown, bf, GM_RESID);
  }
  D.head.rows = c->vocab;
  D.head.cols = d;
  head_plan(D.head, bf);
  D.attn.H = (int32_t)c->n_head;
  D.attn.Hkv = (int32_t)c->n_kv;
  D.attn.hd = (int32_t)c->head_dim;
  D.attn.kv_is_bf16 = c->kv_dtype == LLMK_BF16;
  D.attn.kv_q8 = c->kv_dtype == LLMK_Q8;
  attn_plan(D.attn, c->max_seq);

  int64_t part = 0;
  const GemvParams* gs[4] = {&D.qkv, &D.o, &D.gu, &D.down};
  int ncnt = 0;
  for (int i = 0; i < 4 && !D.rowdot; ++i) {
    const int nacc = (i == 2) ? 2 : 1;
    const int64_t f = gs[i]->ksplit > 1 ? (int64_t)gs[i]->ksplit * nacc * gs[i]->N : 0;
    if (f > part) part = f;
    if (gs[i]->n_cblk > ncnt) ncnt = gs[i]->n_cblk;
  }
  D.n_gemv_counters = ncnt;
  Carve cv(ws);
  D.state = cv.take<DecodeState>(1);
  D.x = cv.take<float>(d);
  D.qkv_buf = cv.take<float>(qd + 2 * kvd);
  D.att = cv.take<float>(qd);
  D.u = cv.take<float>(F);
  D.logits = cv.take<float>(c->vocab);
  D.partial = cv.take<float>(part > 0 ? part : 1);
  D.counters = cv.take<unsigned>(ncnt + c->n_kv + 1);
  D.attn_part = cv.take<float>(attn_part_floats(c->n_head, c->head_dim));
  D.head_val = cv.take<float>(D.head.n_blocks);
  D.head_idx = cv.take<int32_t>(D.head.n_blocks);
  D.tok_scratch = cv.take<int32_t>(kTimeMaxReps);
  D.q8_tok = cv.take<int32_t>(1);
  D.draw1 = cv.take<float>(1);
  D.sampled_tok = cv.take<int32_t>(1);
  D.step_layers = cv.take<StepLayer>(c->n_layer);
  D.step_err = cv.take<int32_t>(4);
  D.step_cnt = cv.take<unsigned>(1);
  D.step_val = cv.take<float>(kStepMaxWG);
  D.step_idx = cv.take<int32_t>(kStepMaxWG);
  auto stride32 = [](int64_t n) { return (n + 31) / 32 * 32; };   // 256-byte aligned versions
  D.step_x_stride = stride32(d);
  D.step_qkv_stride = stride32(qd + 2 * kvd);
  D.step_att_stride = stride32(qd);
  D.step_u_stride = stride32(F);
  const int64_t nx = 2 * c->n_layer * D.step_x_stride, nq = c->n_layer * D.step_qkv_stride;
  const int64_t na = c->n_layer * D.step_att_stride, nu = c->n_layer * D.step_u_stride;
  const int64_t np = attn_part_floats(c->n_head, c->head_dim);
  // activations (4 bytes each, every stride a multiple of 32), then the parts (8 bytes each), contiguous
  D.step_tagged_words = nx + nq + na + nu + 2 * np;
  D.step_tagged = cv.take<uint32_t>(D.step_tagged_words);
  D.step_x = D.step_tagged;
  D.step_qkv = D.step_x + nx;
  D.step_att = D.step_qkv + nq;
  D.step_u = D.step_att + na;
  D.step_part = reinterpret_cast<uint64_t*>(D.step_u + nu);
  D.bytes = cv.off;
}

int64_t counters_total(const llmk_config* c, const DecodePlan& D) { return D.n_gemv_counters + c->n_kv + 1; }

const llmk_tensor& layer_t(const llmk_model* m, int64_t l, int which) { return m->layers[l * LLMK_LAYER_TENSORS + which]; }

int32_t model_check(const llmk_config* c, const llmk_model* m) {
  if (!m || !m->layers) return LLMK_INVALID_ARGUMENT;
  if (!m->emb.ptr || !m->w_out.ptr || !m->g_final.ptr || !m->rope_table.ptr) return LLMK_INVALID_ARGUMENT;
  for (int64_t l = 0; l < c->n_layer; ++l)
    for (int t = 0; t < LLMK_LAYER_TENSORS; ++t)
      if (!layer_t(m, l, t).ptr) return LLMK_INVALID_ARGUMENT;
  return LLMK_OK;
}

int32_t model_lengths(const llmk_config* c, const llmk_model* m) {
  const int64_t d = c->d, qd = c->n_head * c->head_dim, kvd = c->n_kv * c->head_dim, F = c->hidden;
  if (c->w_dtype == LLMK_Q8) {   // q8 packs: byte counts
    if (m->emb.len != c->vocab * d || m->w_out.len != q8_pack_bytes(c->vocab, d) || m->g_final.len != d)
      return LLMK_WEIGHT_LENGTH_MISMATCH;
    if (m->rope_table.len != c->max_seq * c->head_dim) return LLMK_WEIGHT_LENGTH_MISMATCH;
    const int64_t want[LLMK_LAYER_TENSORS] = {q8_pack_bytes(qd, d), q8_pack_bytes(kvd, d), q8_pack_bytes(kvd, d),
                                              q8_pack_bytes(d, qd), q8_pack_bytes(F, d), q8_pack_bytes(F, d),
                                              q8_pack_bytes(d, F), d, d};
    for (int64_t l = 0; l < c->n_layer; ++l)
      for (int t = 0; t < LLMK_LAYER_TENSORS; ++t)
        if (layer_t(m, l, t).len != want[t]) return LLMK_WEIGHT_LENGTH_MISMATCH;
    return LLMK_OK;
  }
  if (m->emb.len != c->vocab * d || m->w_out.len != c->vocab * d || m->g_final.len != d) return LLMK_WEIGHT_LENGTH_MISMATCH;
  if (m->rope_table.len != c->max_seq * c->head_dim) return LLMK_WEIGHT_LENGTH_MISMATCH;
  const int64_t want[LLMK_LAYER_TENSORS] = {d * qd, d * kvd, d * kvd, qd * d, d * F, d * F, F * d, d, d};
  for (int64_t l = 0; l < c->n_layer; ++l)
    for (int t = 0; t < LLMK_LAYER_TENSORS; ++t)
      if (layer_t(m, l, t).len != want[t]) return LLMK_WEIGHT_LENGTH_MISMATCH;
  return LLMK_OK;
}

bool weights_aligned(const llmk_config* c, const llmk_model* m) {
  if (!aligned16(m->emb.ptr) || !aligned16(m->w_out.ptr)) return false;
  for (int64_t l = 0; l < c->n_layer; ++l)
    for (int t = 0; t < LLMK_WDOWN + 1; ++t)
      if (!aligned16(layer_t(m, l, t).ptr)) return false;
  return true;
}

// A decode call advanced `slot` to n_pos positions: the slot record, and the flat-cache records of every
// layer's K and V buffer where the pool keeps them.
void pool_advance(llmk_kv_pool* p, int64_t slot, int64_t n_pos) {
  p->slot_len_h[slot] = n_pos;
  const int64_t row = p->n_kv * p->head_dim;
  for (int64_t l = 0; l < p->n_layer; ++l) {
    if (p->len_k_h) p->len_k_h[l * p->n_slots + slot] = n_pos * row;
    if (p->len_v_h) p->len_v_h[l * p->n_slots + slot] = n_pos * row;
  }
}

int32_t pool_check(const llmk_config* c, const llmk_kv_pool* p) {
  if (!p || !p->k || !p->v || !p->slot_len_h) return LLMK_INVALID_ARGUMENT;
  if (p->n_layer != c->n_layer || p->n_kv != c->n_kv || p->head_dim != c->head_dim || p->dtype != c->kv_dtype)
    return LLMK_INVALID_ARGUMENT;
  for (int64_t l = 0; l < p->n_layer; ++l)
    if (!p->k[l] || !p->v[l]) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({p->n_slots, p->capacity});
  if (st == LLMK_OK && p->pages) st = pages_check(p);
  return st;
}

// Paged pools: reserve the positions the call writes ([begin, end) of each slot); contiguous pools: nothing.
int32_t pool_reserve(llmk_kv_pool* p, const KvReserve* req, int64_t n, hipStream_t s) {
  return p->pages ? pages_reserve(p, req, n, s) : LLMK_OK;
}
int32_t pool_reserve1(llmk_kv_pool* p, int64_t slot, int64_t begin, int64_t end, hipStream_t s) {
  const KvReserve r{slot, begin, end};
  return pool_reserve(p, &r, 1, s);
}
// the positions [pos[r], pos[r] + n) of every row's slot, all or none
int32_t batch_reserve(llmk_kv_pool* p, int64_t B, const int64_t* slots, const int64_t* pos, int64_t n, hipStream_t s) {
  if (!p->pages) return LLMK_OK;
  std::vector<KvReserve> r((size_t)B);
  for (int64_t i = 0; i < B; ++i) r[(size_t)i] = KvReserve{slots[i], pos[i], pos[i] + n};
  return pages_reserve(p, r.data(), B, s);
}

// The kernels of one decode step, in order: per layer K_QKV, K_ATTN, K_O, K_GATEUP, K_DOWN, then K_HEAD.
enum StepKernel { K_QKV = 0, K_ATTN = 1, K_O = 2, K_GATEUP = 3, K_DOWN = 4, K_HEAD = 5, K_CLASSES = 6,
                  K_STEP = 6 /* the persistent step kernel (timing aid only) */ };

// Launch kernel `which` of layer l (K_HEAD: the tail, l ignored). Token and position are read from D.state.
hipError_t launch_kernel(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, int64_t slot,
                         DecodePlan& D, int64_t l, int which, float* logits, int32_t* token_out, float* hidden,
                         hipStream_t s) {
  const int bf = c->w_dtype == LLMK_BF16;
  const int64_t d = c->d, kvd = c->n_kv * c->head_dim;
  const int64_t kv_off = pool->pages ? 0 : slot * pool->capacity * kvd;
  const int64_t kvsz = dtype_size(c->kv_dtype);
  unsigned* gcnt = D.counters;
  unsigned* acnt = D.counters + D.n_gemv_counters;
  unsigned* hcnt = acnt + c->n_kv;
  if (which == K_HEAD && D.q8) {
    // logits = W_out rmsnorm(x) g_final over the int8 head, then the greedy token and the state's advance
    RowdotParams h = D.rhead;
    h.w0 = m->w_out.ptr;
    h.in = D.x;
    h.in_is_w = 0;
    h.in_state = nullptr;
    h.gain = static_cast<const float*>(m->g_final.ptr);
    h.eps = (float)c->eps;
    h.y = logits ? logits : D.logits;
    hipError_t e = rowdot_q8_launch(h, GM_PLAIN, s);
    const int32_t bpr = std::min<int32_t>(D.head.n_blocks, 128);
    if (e == hipSuccess)
      e = argmax_launch(h.y, 1, c->vocab, D.q8_tok, nullptr, D.head_val, D.head_idx, hcnt, bpr, s);
    if (e == hipSuccess) e = state_advance_launch(D.state, D.q8_tok, token_out, s);
    return e;
  }
  if (which == K_HEAD) {
    // logits = W_out rmsnorm(x) g_final; greedy token; state advances
    HeadParams h = D.head;
    h.w = m->w_out.ptr;
    h.x = D.x;
    h.gain = static_cast<const float*>(m->g_final.ptr);
    h.eps = (float)c->eps;
    h.y = logits ? logits : D.logits;
    h.part_val = D.head_val;
    h.part_idx = D.head_idx;
    h.counter = hcnt;
    h.token_out = token_out;
    h.logit_out = nullptr;
    h.state = D.state;
    return head_launch(h, bf, s);
  }
  const float* g_attn = static_cast<const float*>(layer_t(m, l, LLMK_GATTN).ptr);
  const float* g_ffn = static_cast<const float*>(layer_t(m, l, LLMK_GFFN).ptr);
  if (which == K_ATTN) {
    // RoPE on q and k, append k, v at pos, attention over positions 0..pos of this slot
    AttnParams a = D.attn;
    a.q = nullptr;
    a.qkv_raw = D.qkv_buf;
    a.k = static_cast<const char*>(pool->k[l]) + kv_off * kvsz;
    a.v = static_cast<const char*>(pool->v[l]) + kv_off * kvsz;
    a.k_w = static_cast<char*>(pool->k[l]) + kv_off * kvsz;
    a.v_w = static_cast<char*>(pool->v[l]) + kv_off * kvsz;
    if (a.kv_q8) {   // the slot's scales (kv_off / head_dim rows of scales in)
      a.k_scale_w = pool_scales(pool, pool->k[l]) + kv_off / c->head_dim;
      a.v_scale_w = pool_scales(pool, pool->v[l]) + kv_off / c->head_dim;
      a.k_scale = a.k_scale_w;
      a.v_scale = a.v_scale_w;
    }
    a.pg = pages_view(pool);
    a.pg.table = pages_slot_row(pool, slot);
    a.rope_table = static_cast<const float*>(m->rope_table.ptr);
    a.rope_layout = c->rope_layout;
    a.state = D.state;
    a.ctx = 0;
    a.part = D.attn_part;
    a.counters = acnt;
    a.out = D.att;
    return attn_launch(a, s);
  }
  if (D.rowdot) {
    switch (which) {
      case K_QKV: {   // h = rmsnorm(x) g_attn;  q|k|v = h W  (raw; layer 0 reads x = emb[token])
        RowdotParams r = D.rqkv;
        r.w0 = layer_t(m, l, LLMK_WQ).ptr;
        r.w1 = layer_t(m, l, LLMK_WK).ptr;
        r.w2 = layer_t(m, l, LLMK_WV).ptr;
        if (l == 0) { r.in = m->emb.ptr; r.in_is_w = 1; r.in_state = D.state; }
        else { r.in = D.x; r.in_is_w = 0; r.in_state = nullptr; }
        r.gain = g_attn;
        r.eps = (float)c->eps;
        r.y = D.qkv_buf;
        return D.q8 ? rowdot_q8_launch(r, GM_QKV, s) : rowdot_launch(r, GM_QKV, bf, s);
      }
      case K_O: {     // x = x + att Wo   (layer 0: x = emb[token] + att Wo)
        RowdotParams o = D.ro;
        o.w0 = layer_t(m, l, LLMK_WO).ptr;
        o.in = D.att;
        o.x = D.x;
        if (l == 0) { o.base = m->emb.ptr; o.base_is_w = 1; o.base_state = D.state; }
        else { o.base = D.x; o.base_is_w = 0; o.base_state = nullptr; }
        return D.q8 ? rowdot_q8_launch(o, GM_RESID, s) : rowdot_launch(o, GM_RESID, bf, s);
      }
      case K_GATEUP: {   // h = rmsnorm(x) g_ffn;  u = silu(h Wgate) * (h Wup)
        RowdotParams gu = D.rgu;
        gu.w0 = layer_t(m, l, LLMK_WGATE).ptr;
        gu.w1 = layer_t(m, l, LLMK_WUP).ptr;
        gu.in = D.x;
        gu.gain = g_ffn;
        gu.eps = (float)c->eps;
        gu.y = D.u;
        return D.q8 ? rowdot_q8_launch(gu, GM_GATEUP, s) : rowdot_launch(gu, GM_GATEUP, bf, s);
      }
      case K_DOWN: {  // x = x + u Wdown
        RowdotParams dn = D.rdown;
        dn.w0 = layer_t(m, l, LLMK_WDOWN).ptr;
        dn.in = D.u;
        dn.x = D.x;
        dn.base = D.x;
        dn.hidden = hidden ? hidden + l * d : nullptr;
        return D.q8 ? rowdot_q8_launch(dn, GM_RESID, s) : rowdot_launch(dn, GM_RESID, bf, s);
      }
    }
    return hipErrorInvalidValue;
  }
  switch (which) {
    case K_QKV: {
      GemvParams g = D.qkv;
      g.w0 = layer_t(m, l, LLMK_WQ).ptr;
      g.w1 = layer_t(m, l, LLMK_WK).ptr;
      g.w2 = layer_t(m, l, LLMK_WV).ptr;
      if (l == 0) { g.in = m->emb.ptr; g.in_is_w = 1; g.in_state = D.state; }
      else { g.in = D.x; g.in_is_w = 0; g.in_state = nullptr; }
      g.gain = g_attn;
      g.eps = (float)c->eps;
      g.partial = D.partial;
      g.counters = gcnt;
      g.y = D.qkv_buf;
      return gemv_launch(g, GM_QKV, bf, 0, s);
    }
    case K_O: {
      GemvParams o = D.o;
      o.w0 = layer_t(m, l, LLMK_WO).ptr;
      o.in = D.att;
      o.in_is_w = 0;
      o.gain = nullptr;
      o.partial = D.partial;
      o.counters = gcnt;
      o.x = D.x;
      if (l == 0) { o.base = m->emb.ptr; o.base_is_w = 1; o.base_state = D.state; }
      else { o.base = D.x; o.base_is_w = 0; o.base_state = nullptr; }
      o.hidden = nullptr;
      return gemv_launch(o, GM_RESID, bf, 0, s);
    }
    case K_GATEUP: {
      GemvParams gu = D.gu;
      gu.w0 = layer_t(m, l, LLMK_WGATE).ptr;
      gu.w1 = layer_t(m, l, LLMK_WUP).ptr;
      gu.in = D.x;
      gu.in_is_w = 0;
      gu.gain = g_ffn;
      gu.eps = (float)c->eps;
      gu.partial = D.partial;
      gu.counters = gcnt;
      gu.y = D.u;
      return gemv_launch(gu, GM_GATEUP, bf, 0, s);
    }
    case K_DOWN: {
      GemvParams dn = D.down;
      dn.w0 = layer_t(m, l, LLMK_WDOWN).ptr;
      dn.in = D.u;
      dn.in_is_w = 0;
      dn.gain = nullptr;
      dn.partial = D.partial;
      dn.counters = gcnt;
      dn.x = D.x;
      dn.base = D.x;
      dn.base_is_w = 0;
      dn.hidden = hidden ? hidden + l * d : nullptr;
      return gemv_launch(dn, GM_RESID, bf, 0, s);
    }
  }
  return hipErrorInvalidValue;
}

// Enqueue one decode step's kernels. With ev, event 2k is recorded before and 2k+1 after kernel k, on the
// kernels' own stream.
hipError_t enqueue_step(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, int64_t slot,
                        DecodePlan& D, float* logits, int32_t* token_out, float* hidden, hipStream_t s,
                        hipEvent_t* ev = nullptr) {
  int kidx = 0;
  auto one = [&](int64_t l, int which) -> hipError_t {
    hipError_t e = ev ? hipEventRecord(ev[2 * kidx], s) : hipSuccess;
    if (e == hipSuccess) e = launch_kernel(c, m, pool, slot, D, l, which, logits, token_out, hidden, s);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2 * kidx + 1], s);
    ++kidx;
    return e;
  };
  hipError_t e = hipSuccess;
  for (int64_t l = 0; l < c->n_layer && e == hipSuccess; ++l)
    for (int k = K_QKV; k <= K_DOWN && e == hipSuccess; ++k) e = one(l, k);
  if (e == hipSuccess) e = one(0, K_HEAD);
  return e;
}

// ---- the persistent step ----

// Whether the persistent step supports this shape (device aside): bf16 output-major weights, rows a whole
// number of 16-byte loads, every projection input within the LDS it stages into, at most 8 query heads per
// K/V head (the attention block's limit).
bool step_shape_ok(const llmk_config* c, int nwg) {
  const int64_t qd = c->n_head * c->head_dim;
  if (c->w_layout != LLMK_W_OUT_IN || c->n_layer > STEP_MAX_LAYERS) return false;
  if (c->w_dtype != LLMK_BF16 && c->w_dtype != LLMK_Q8) return false;
  // int8 packs: every projection input in whole groups of LLMK_Q8_GROUP (config_check), head dims 64 .. 256
  if (c->w_dtype == LLMK_Q8 && (c->head_dim < 64 || c->kv_dtype == LLMK_Q8)) return false;
  if (c->d % 8 || qd % 8 || c->hidden % 8) return false;
  if (std::max(std::max(c->d, qd), c->hidden) > STEP_MAX_VIN) return false;
  if (c->n_head / c->n_kv > 8) return false;
  if (nwg <= 0) return false;
  // a workgroup's rows of each projection: the residual rows it keeps, and at most STEP_MAX_WAVE_ROWS a wave
  auto most = [nwg](int64_t n) { return (n + nwg - 1) / nwg; };
  const int64_t kvd = c->n_kv * c->head_dim, wg_rows = (int64_t)STEP_MAX_WAVE_ROWS * 8;
  if (most(c->d) > STEP_MAX_RES) return false;
  return most(qd) + 2 * most(kvd) <= wg_rows && 2 * most(c->hidden) <= wg_rows && most(c->vocab) <= wg_rows;
}

// Workgroups of the persistent step for this call (0: run one kernel per operation). -1: refused.
int step_workgroups(const llmk_config* c) {
  if (c->step_path == LLMK_STEP_PER_OP || c->kv_dtype == LLMK_Q8) return 0;   // the int8 cache: per operation
  int nwg = step_grid(c->kv_dtype == LLMK_BF16, (int)c->head_dim, c->w_dtype == LLMK_Q8);
  if (nwg > kStepMaxWG || !step_shape_ok(c, nwg)) nwg = 0;
  if (nwg == 0 && c->step_path == LLMK_STEP_PERSISTENT) return -1;
  return nwg;
}

// Prelude of a persistent call: zero the tickets, the error flag and the tagged activations, set the
// state, fill the layer table.
hipError_t step_prelude(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, DecodePlan& D,
                        int32_t token, int32_t pos, hipStream_t s) {
  hipError_t e = fill_u32_launch(D.step_cnt, 1, 0u, s);
  if (e == hipSuccess) e = fill_u32_launch(reinterpret_cast<unsigned*>(D.step_err), 4, 0u, s);
  if (e == hipSuccess) e = fill_u32_launch(D.step_tagged, D.step_tagged_words, 0u, s);
  if (e == hipSuccess) e = set_state_launch(D.state, token, pos, s);
  for (int64_t l0 = 0; e == hipSuccess && l0 < c->n_layer; l0 += 8) {
    StepTableChunk ch{};
    ch.first = (int32_t)l0;
    ch.count = (int32_t)std::min<int64_t>(8, c->n_layer - l0);
    for (int32_t j = 0; j < ch.count; ++j) {
      StepLayer& L = ch.layers[j];
      const int64_t l = l0 + j;
      const int ws[7] = {LLMK_WQ, LLMK_WK, LLMK_WV, LLMK_WO, LLMK_WGATE, LLMK_WUP, LLMK_WDOWN};
      for (int t = 0; t < 7; ++t) L.w[t] = static_cast<const bf16_t*>(layer_t(m, l, ws[t]).ptr);
      L.g1 = static_cast<const float*>(layer_t(m, l, LLMK_GATTN).ptr);
      L.g2 = static_cast<const float*>(layer_t(m, l, LLMK_GFFN).ptr);
      L.k = pool->k[l];
      L.v = pool->v[l];
    }
    e = step_table_launch(D.step_layers, ch, s);
  }
  return e;
}

StepParams step_params(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, int64_t slot,
                       DecodePlan& D, int nwg, float* logits, float* hidden, int32_t* token_out) {
  StepParams p{};
  p.layers = D.step_layers;
  p.emb = static_cast<const bf16_t*>(m->emb.ptr);
  p.w_out = static_cast<const bf16_t*>(m->w_out.ptr);
  p.g_final = static_cast<const float*>(m->g_final.ptr);
  p.rope_table = static_cast<const float*>(m->rope_table.ptr);
  p.n_layer = (int32_t)c->n_layer;
  p.d = (int32_t)c->d;
  p.qd = (int32_t)(c->n_head * c->head_dim);
  p.kvd = (int32_t)(c->n_kv * c->head_dim);
  p.F = (int32_t)c->hidden;
  p.V = (int32_t)c->vocab;
  p.H = (int32_t)c->n_head;
  p.Hkv = (int32_t)c->n_kv;
  p.hd = (int32_t)c->head_dim;
  p.rope_layout = c->rope_layout;
  p.eps = (float)c->eps;
  p.nwg = nwg;
  p.kv_off = pool->pages ? 0 : slot * pool->capacity * c->n_kv * c->head_dim;
  p.kv_table = pages_slot_row(pool, slot);
  p.kv_shift = pages_shift(pool);
  p.attn_chunk = D.attn.chunk;
  p.state = D.state;
  p.x = D.step_x;
  p.qkv = D.step_qkv;
  p.att = D.step_att;
  p.u = D.step_u;
  p.x_stride = D.step_x_stride;
  p.qkv_stride = D.step_qkv_stride;
  p.att_stride = D.step_att_stride;
  p.u_stride = D.step_u_stride;
  p.attn_part = D.step_part;
  p.logits = logits;
  p.hidden = hidden;
  p.head_val = D.step_val;
  p.head_idx = D.step_idx;
  p.head_cnt = D.step_cnt;
  p.err = D.step_err;
  p.token_out = token_out;
  p.give_up = (c->test_flags & LLMK_TEST_WAIT_GIVE_UP) ? 1 : 0;
  p.qw = c->w_dtype == LLMK_Q8 ? 1 : 0;
  return p;
}

// llmk_decode_kernel_time for the persistent step kernel: `reps` steps from (token, pos) as one captured
// launch replayed between two events, then the ordinary step at (token, pos) again.
int32_t time_step_kernel(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                         int64_t token, int64_t pos, int32_t reps, int32_t* token_out, float* ms_per_launch_h,
                         DecodePlan& D, hipStream_t s) {
  const int nwg = step_workgroups(cfg);
  if (nwg <= 0) return LLMK_INVALID_ARGUMENT;
  if (pos + reps > pool->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = step_prelude(cfg, model, pool, D, (int32_t)token, (int32_t)pos, s);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t ee = step_launch(step_params(cfg, model, pool, slot, D, nwg, nullptr, nullptr, D.tok_scratch),
                                cfg->kv_dtype == LLMK_BF16, cs);
    e = hipStreamEndCapture(cs, &graph);
    if (ee != hipSuccess) e = ee;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int32_t r = 0; e == hipSuccess && r < reps; ++r) e = hipGraphLaunch(exec, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  int32_t err = 0;
  if (e == hipSuccess) e = hipMemcpy(&err, D.step_err, sizeof(err), hipMemcpyDeviceToHost);
  // the ordinary step at (token, pos): the K/V at pos and token_out as llmk_decode_step leaves them
  if (e == hipSuccess) e = step_prelude(cfg, model, pool, D, (int32_t)token, (int32_t)pos, s);
  if (e == hipSuccess)
    e = step_launch(step_params(cfg, model, pool, slot, D, nwg, nullptr, nullptr, token_out), cfg->kv_dtype == LLMK_BF16, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (cs) (void)hipStreamDestroy(cs);
  if (e != hipSuccess || err != 0) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos + 1);
  *ms_per_launch_h = ms / (float)reps;
  return LLMK_OK;
}

// Common checks of decode_step / decode_steps, in the documented order.
int32_t decode_checks(const llmk_config* cfg, const llmk_model* model, const llmk_kv_pool* pool, int64_t slot,
                      int64_t token, int64_t pos, int64_t n_steps, const void* out_ptr, const void* ws) {
  if (!cfg || !model || !pool || !out_ptr || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if ((st = model_check(cfg, model)) != LLMK_OK) return st;
  if ((st = model_lengths(cfg, model)) != LLMK_OK) return st;
  if ((st = pool_check(cfg, pool)) != LLMK_OK) return st;
  if (!weights_aligned(cfg, model)) return LLMK_INVALID_ARGUMENT;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  if (token < 0 || token >= cfg->vocab) return LLMK_TOKEN_OUT_OF_RANGE;
  if (pos < 0 || pos + n_steps > cfg->max_seq) return LLMK_POSITION_OUT_OF_RANGE;
  if (pos != pool->slot_len_h[slot]) return LLMK_CACHE_LENGTH_MISMATCH;
  if (pos + n_steps > pool->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  return LLMK_OK;
}

// ---- batched decode ------------------------------------------------------------------------------------

constexpr int kBatchTargetBlocks = 256;   // workgroups a row GEMM aims for (K is split up to that); measured 128,
                                          // 192, 256, 384 (64-row 8B step: 14.62, 13.89, 12.55, 13.22 ms)
constexpr int kBatchAttnTilesPerPart = 20;   // measured 12, 16, 20, 24, 28, 32 (64-row 8B step: 13.63, 12.75, 12.48, 13.61, 12.62, 12.62 ms)

struct BatchPlan {
  int64_t B = 0;
  int64_t qkv_n = 0;                    // q|k|v row length (H + 2 Hkv) hd
  AttnParams attn{};
  BatchState* state = nullptr;
  float* x = nullptr;                   // [B][d] residual stream
  bf16_t* h_hi = nullptr;               // [B][max(d)] normed input of q|k|v, gate|up and the head
  bf16_t* h_lo = nullptr;
  float* qkv_buf = nullptr;             // [B][(H + 2 Hkv) hd] raw q|k|v
  bf16_t* att_hi = nullptr;             // [B][H hd]
  bf16_t* att_lo = nullptr;
  bf16_t* u_hi = nullptr;               // [B][F]
  bf16_t* u_lo = nullptr;
  unsigned* counters = nullptr;         // B * Hkv attention tickets, then B head-argmax tickets
  float* attn_part = nullptr;
  int32_t* tok_scratch = nullptr;       // kTimeMaxReps * B tokens: repeated timing launches of the head
  int64_t bytes = 0;
  bool prefill = false;                 // rows of one chunk: K/V appended for all rows before any attends
  // the decode batch's q|k|v, o, gate|up and down as tiled matrix-core GEMMs (their split partials in py)
  PgemmParams pqkv{}, po{}, pgu{}, pdown{}, phead{};
  float* py = nullptr;
  float* hlogits = nullptr;             // [B][vocab] when the caller takes no logits
  int32_t* htok = nullptr;              // [B] greedy tokens of the step
  float* hval = nullptr;                // the row argmax's partials and tickets
  int32_t* hidx = nullptr;
  unsigned* hcnt = nullptr;
  int32_t hbpr = 0;
};

// The batched path runs bf16 weights in the output-major layout (matrix-core operands).
bool batch_config_ok(const llmk_config* c) { return c->w_dtype == LLMK_BF16 && c->w_layout == LLMK_W_OUT_IN; }

void plan_batch(const llmk_config* c, int64_t B, void* ws, BatchPlan& P, bool row_gemms = true) {
  const int64_t d = c->d, qd = c->n_head * c->head_dim, kvd = c->n_kv * c->head_dim, F = c->hidden;
  P.B = B;
  P.qkv_n = qd + 2 * kvd;
  P.attn.H = (int32_t)c->n_head;
  P.attn.Hkv = (int32_t)c->n_kv;
  P.attn.hd = (int32_t)c->head_dim;
  P.attn.kv_is_bf16 = c->kv_dtype == LLMK_BF16;
  P.attn.kv_q8 = c->kv_dtype == LLMK_Q8;
  // every row of the batch brings its own (row, K/V head) pairs, so parts can be long: about 16 tiles each
  // (measured on the 64-row, 8,320-position pool, us per layer: 312 at the batch-1 split, 299 at 6 tiles, 261
  // at 10, 235 at 16, 261 at 24, 357 at 40)
  attn_plan(P.attn, c->max_seq, kBatchAttnTilesPerPart);
  P.attn.rows = (int32_t)B;

  Carve cv(ws);
  P.state = cv.take<BatchState>(1);
  P.x = cv.take<float>(B * d);
  P.h_hi = cv.take<bf16_t>(B * d);
  P.h_lo = cv.take<bf16_t>(B * d);
  P.qkv_buf = cv.take<float>(B * (qd + 2 * kvd));
  P.att_hi = cv.take<bf16_t>(B * qd);
  P.att_lo = cv.take<bf16_t>(B * qd);
  P.u_hi = cv.take<bf16_t>(B * F);
  P.u_lo = cv.take<bf16_t>(B * F);
  P.counters = cv.take<unsigned>(B * c->n_kv + B);
  P.attn_part = cv.take<float>(B * (int64_t)P.attn.n_parts * c->n_head * (c->head_dim + 2));
  P.tok_scratch = cv.take<int32_t>(kTimeMaxReps * B);
  if (row_gemms) {
    // the same tiled GEMM as prefill: with 64 rows it re-reads the activations from L2 less than the skinny
    // kernel does (measured on the 8B shape, 64 rows: q|k|v 42 -> 30 us, o 41 -> 22, gate|up 114 -> 85,
    // down 74 -> 48)
    PgemmParams* g4[4] = {&P.pqkv, &P.po, &P.pgu, &P.pdown};
    const int64_t N4[4] = {qd + 2 * kvd, d, 2 * F, d};
    const int64_t K4[4] = {d, qd, d, F};
    int64_t yfl = 0;
    for (int i = 0; i < 4; ++i) {
      g4[i]->M = (int32_t)B;
      g4[i]->N = N4[i];
      g4[i]->K = K4[i];
      g4[i]->lda = K4[i];
      g4[i]->n0 = N4[i];
      pgemm_plan(*g4[i], kBatchTargetBlocks);
      yfl = std::max(yfl, (int64_t)g4[i]->ksplit * B * N4[i]);
    }
    P.pqkv.n0 = qd;
    P.pqkv.n1 = kvd;
    P.pgu.n0 = F;
    P.pgu.n1 = F;
    P.py = cv.take<float>(yfl);
    // the head: one split into the logits, then a row argmax (tickets reset by its last block)
    P.phead.M = (int32_t)B;
    P.phead.N = c->vocab;
    P.phead.K = d;
    P.phead.lda = d;
    P.phead.n0 = c->vocab;
    pgemm_plan(P.phead, 1);
    P.hlogits = cv.take<float>(B * c->vocab);
    P.htok = cv.take<int32_t>(B);
    P.hbpr = c->vocab >= 65536 ? 64 : (int32_t)((c->vocab + 1023) / 1024);
    P.hval = cv.take<float>(B * P.hbpr);
    P.hidx = cv.take<int32_t>(B * P.hbpr);
    P.hcnt = P.counters ? P.counters + B * c->n_kv : nullptr;
  }
  P.bytes = cv.off;
}

int64_t batch_counters_total(const llmk_config* c, const BatchPlan& P) {
  return P.B * c->n_kv + P.B;
}

// The kernels of one batched step, in order: per layer BK_NORM1, BK_QKV, BK_ATTN, BK_O, BK_NORM2, BK_GATEUP,
// BK_DOWN, then BK_NORMF and BK_HEAD.
enum BatchKernel { BK_NORM1 = 0, BK_QKV, BK_ATTN, BK_O, BK_NORM2, BK_GATEUP, BK_DOWN, BK_NORMF, BK_HEAD, BK_CLASSES };

// Launch kernel `which` of layer l of a batched step (BK_NORMF / BK_HEAD: the tail, l ignored); tokens,
// positions and slots are read from P.state on the device.
hipError_t launch_batch_kernel(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, BatchPlan& P,
                               int64_t l, int which, float* logits, int32_t* tokens_out, float* hidden,
                               hipStream_t s) {
  const int64_t d = c->d, kvd = c->n_kv * c->head_dim;
  const int32_t B = (int32_t)P.B;
  const float eps = (float)c->eps;
  switch (which) {
    case BK_NORM1:   // h = rmsnorm(x) g_attn (layer 0: x = emb[token] first)
      return bnorm_launch(P.x, l == 0 ? m->emb.ptr : nullptr, 1, P.state, B, d,
                          static_cast<const float*>(layer_t(m, l, LLMK_GATTN).ptr), eps, P.h_hi, P.h_lo, s);
    case BK_QKV: {   // q|k|v = W h
      PgemmParams g = P.pqkv;
      g.ahi = P.h_hi;
      g.alo = P.h_lo;
      g.w0 = layer_t(m, l, LLMK_WQ).ptr;
      g.w1 = layer_t(m, l, LLMK_WK).ptr;
      g.w2 = layer_t(m, l, LLMK_WV).ptr;
      g.y = P.py;
      g.out = P.qkv_buf;
      g.ldo = g.N;
      return pgemm_launch(g, PG_STORE, s);
    }
    case BK_ATTN: {  // RoPE, K/V append at each row's position in its slot, attention over the row's context
      AttnParams a = P.attn;
      a.q = nullptr;
      a.qkv_raw = P.qkv_buf;
      a.qkv_stride = P.qkv_n;
      a.k = pool->k[l];
      a.v = pool->v[l];
      a.k_w = pool->k[l];
      a.v_w = pool->v[l];
      a.slot_elems = pool->capacity * kvd;
      a.pg = pages_view(pool);
      if (a.kv_q8) {
        a.k_scale_w = pool_scales(pool, pool->k[l]);
        a.v_scale_w = pool_scales(pool, pool->v[l]);
        a.k_scale = a.k_scale_w;
        a.v_scale = a.v_scale_w;
      }
      a.rope_table = static_cast<const float*>(m->rope_table.ptr);
      a.rope_layout = c->rope_layout;
      a.state = nullptr;
      a.bstate = P.state;
      a.part = P.attn_part;
      a.counters = P.counters;
      a.out = nullptr;
      a.out_hi = P.att_hi;
      a.out_lo = P.att_lo;
      a.no_append = P.prefill ? 1 : 0;
      if (P.prefill) {
        hipError_t e = rope_append_rows_launch(P.qkv_buf, P.qkv_n, P.state, B, a.H, a.Hkv, a.hd, a.rope_table,
                                               a.rope_layout, pool->k[l], pool->v[l], c->kv_dtype, a.slot_elems, a.pg,
                                               a.k_scale_w, a.v_scale_w, s);
        if (e != hipSuccess) return e;
      }
      return attn_launch(a, s);
    }
    case BK_O: {     // x += Wo att
      PgemmParams g = P.po;
      g.ahi = P.att_hi;
      g.alo = P.att_lo;
      g.w0 = layer_t(m, l, LLMK_WO).ptr;
      g.y = P.py;
      g.out = P.x;
      g.ldo = d;
      return pgemm_launch(g, PG_RESID, s);
    }
    case BK_NORM2:   // h = rmsnorm(x) g_ffn
      return bnorm_launch(P.x, nullptr, 1, P.state, B, d, static_cast<const float*>(layer_t(m, l, LLMK_GFFN).ptr),
                          eps, P.h_hi, P.h_lo, s);
    case BK_GATEUP: {   // u = silu(Wg h) * (Wu h)
      PgemmParams g = P.pgu;
      g.ahi = P.h_hi;
      g.alo = P.h_lo;
      g.w0 = layer_t(m, l, LLMK_WGATE).ptr;
      g.w1 = layer_t(m, l, LLMK_WUP).ptr;
      g.y = P.py;
      g.uhi = P.u_hi;
      g.ulo = P.u_lo;
      return pgemm_launch(g, PG_GATEUP, s);
    }
    case BK_DOWN: {  // x += Wd u
      PgemmParams g = P.pdown;
      g.ahi = P.u_hi;
      g.alo = P.u_lo;
      g.w0 = layer_t(m, l, LLMK_WDOWN).ptr;
      g.y = P.py;
      g.out = P.x;
      g.ldo = d;
      g.hidden = hidden ? hidden + l * d : nullptr;
      g.hidden_stride = c->n_layer * d;
      return pgemm_launch(g, PG_RESID, s);
    }
    case BK_NORMF:
      return bnorm_launch(P.x, nullptr, 1, P.state, B, d, static_cast<const float*>(m->g_final.ptr), eps, P.h_hi,
                          P.h_lo, s);
    case BK_HEAD: {  // logits = W_out h; greedy token per row; state advances
      if (!P.py) return hipErrorInvalidValue;   // planned without the row GEMMs (prefill has its own head)
      PgemmParams g = P.phead;
      g.ahi = P.h_hi;
      g.alo = P.h_lo;
      g.w0 = m->w_out.ptr;
      g.y = logits ? logits : P.hlogits;
      hipError_t e = pgemm_launch(g, PG_NONE, s);
      if (e == hipSuccess) e = argmax_launch(g.y, B, c->vocab, P.htok, nullptr, P.hval, P.hidx, P.hcnt, P.hbpr, s);
      if (e == hipSuccess) e = batch_advance_launch(P.state, P.htok, tokens_out, B, s);
      return e;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t enqueue_batch(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, BatchPlan& P,
                         float* logits, int32_t* tokens_out, float* hidden, hipStream_t s) {
  hipError_t e = hipSuccess;
  for (int64_t l = 0; l < c->n_layer && e == hipSuccess; ++l)
    for (int k = BK_NORM1; k <= BK_DOWN && e == hipSuccess; ++k)
      e = launch_batch_kernel(c, m, pool, P, l, k, logits, tokens_out, hidden, s);
  if (e == hipSuccess) e = launch_batch_kernel(c, m, pool, P, 0, BK_NORMF, logits, tokens_out, hidden, s);
  if (e == hipSuccess) e = launch_batch_kernel(c, m, pool, P, 0, BK_HEAD, logits, tokens_out, hidden, s);
  return e;
}

// ---- prefill ------------------------------------------------------------------------------------------

constexpr int64_t kPrefillRows = 256;   // rows per chunk: each weight tile serves up to 256 rows

// A chunk of M prompt rows: the batched plan's row buffers, attention and norms, plus the chunk's projections
// (tiled matrix-core GEMMs), their split partials (also the head's logits [M][vocab]) and the argmax partials.
struct PrefillPlan {
  BatchPlan rows;
  PgemmParams qkv{}, o{}, gu{}, down{}, head{};
  float* y = nullptr;
  float* am_val = nullptr;
  int32_t* am_idx = nullptr;
  unsigned* am_cnt = nullptr;
  float* am_logit = nullptr;
  int32_t am_bpr = 0;
  float* hidden = nullptr;              // [M][n_layer][d]: the last chunk's hidden states, when asked for
  float* fa_part = nullptr;             // chunk attention parts (when the shape takes the chunk attention)
  int32_t fa_parts = 0;
  int64_t bytes = 0;
};

void plan_prefill(const llmk_config* c, int64_t M, void* ws, PrefillPlan& P) {
  const int64_t d = c->d, qd = c->n_head * c->head_dim, kvd = c->n_kv * c->head_dim, F = c->hidden;
  plan_batch(c, M, ws, P.rows, false);
  P.rows.prefill = true;
  PgemmParams* gs[5] = {&P.qkv, &P.o, &P.gu, &P.down, &P.head};
  const int64_t Ns[5] = {qd + 2 * kvd, d, 2 * F, d, c->vocab};
  const int64_t Ks[5] = {d, qd, d, F, d};
  int64_t yfl = 0;
  for (int i = 0; i < 5; ++i) {
    gs[i]->M = (int32_t)M;
    gs[i]->N = Ns[i];
    gs[i]->K = Ks[i];
    gs[i]->lda = Ks[i];
    gs[i]->n0 = Ns[i];
    pgemm_plan(*gs[i], i == 4 ? 1 : kBatchTargetBlocks);   // the head: one split, its partial is the logits
    yfl = std::max(yfl, (int64_t)gs[i]->ksplit * M * Ns[i]);
  }
  P.qkv.n0 = qd;
  P.qkv.n1 = kvd;
  P.gu.n0 = F;
  P.gu.n1 = F;
  Carve cv(ws);
  cv.off = P.rows.bytes;
  P.y = cv.take<float>(yfl);
  P.am_bpr = c->vocab >= 65536 ? 64 : (int32_t)((c->vocab + 1023) / 1024);
  P.am_val = cv.take<float>(M * P.am_bpr);
  P.am_idx = cv.take<int32_t>(M * P.am_bpr);
  P.am_cnt = cv.take<unsigned>(M);
  P.am_logit = cv.take<float>(M);
  P.hidden = cv.take<float>(M * c->n_layer * d);
  if (c->kv_dtype != LLMK_Q8 && fattn_supported(c->n_head, c->n_kv, c->head_dim, c->max_seq)) {
    P.fa_parts = (int32_t)fattn_parts(c->max_seq);
    P.fa_part = cv.take<float>(M * c->n_head * P.fa_parts * (c->head_dim + 2));
  }
  P.bytes = cv.off;
}

int64_t prefill_bytes(const llmk_config* c, int64_t n) {
  const int64_t rows = std::min(n, kPrefillRows);
  PrefillPlan P;
  plan_prefill(c, rows, nullptr, P);
  int64_t bytes = P.bytes;
  if (n % rows != 0) {
    plan_prefill(c, n % rows, nullptr, P);
    bytes = std::max(bytes, P.bytes);
  }
  return bytes;
}

// Measurement aid: HIP events recorded on the stream at the phase boundaries of a prefill; a phase's time is
// the span between the event before it and the event after it.
enum PrefillPhase { PF_NORM = 0, PF_PROJ = 1, PF_ATTN = 2, PF_HEAD = 3, PF_CLASSES = 4 };
struct PhaseTimer {
  hipStream_t s = nullptr;
  std::vector<hipEvent_t> ev;
  std::vector<int> cls;                 // cls[i]: the phase that event i closes (-1: a starting mark)
  hipError_t err = hipSuccess;
  void mark(int phase) {
    hipEvent_t e = nullptr;
    if (err == hipSuccess) err = hipEventCreate(&e);
    if (err == hipSuccess) err = hipEventRecord(e, s);
    if (e) {
      ev.push_back(e);
      cls.push_back(phase);
    }
  }
  ~PhaseTimer() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

// One chunk: rows r = 0..M-1 of P at positions state.pos[r] of one slot, through every layer and the head.
hipError_t enqueue_prefill_chunk(const llmk_config* c, const llmk_model* m, const llmk_kv_pool* pool, PrefillPlan& P,
                                 int64_t ctx_end, int32_t* tokens_out, bool want_hidden, hipStream_t s,
                                 PhaseTimer* tm) {
  const int64_t d = c->d;
  BatchPlan& B = P.rows;
  hipError_t e = hipSuccess;
  auto mark = [&](int phase) {
    if (tm && e == hipSuccess) tm->mark(phase);
  };
  mark(-1);
  for (int64_t l = 0; l < c->n_layer && e == hipSuccess; ++l) {
    e = launch_batch_kernel(c, m, pool, B, l, BK_NORM1, nullptr, nullptr, nullptr, s);
    mark(PF_NORM);
    if (e == hipSuccess) {
      PgemmParams g = P.qkv;
      g.ahi = B.h_hi;
      g.alo = B.h_lo;
      g.w0 = layer_t(m, l, LLMK_WQ).ptr;
      g.w1 = layer_t(m, l, LLMK_WK).ptr;
      g.w2 = layer_t(m, l, LLMK_WV).ptr;
      g.y = P.y;
      g.out = B.qkv_buf;
      g.ldo = g.N;
      e = pgemm_launch(g, PG_STORE, s);
    }
    mark(PF_PROJ);
    if (e == hipSuccess && P.fa_part) {   // the chunk's K/V first, then attention of all rows together
      FattnParams a{};
      a.qkv = B.qkv_buf;
      a.qkv_stride = P.qkv.N;
      a.st = B.state;
      a.rows = P.qkv.M;
      a.H = (int32_t)c->n_head;
      a.Hkv = (int32_t)c->n_kv;
      a.k = pool->k[l];
      a.v = pool->v[l];
      a.kv_is_bf16 = c->kv_dtype == LLMK_BF16;
      a.slot_elems = pool->capacity * c->n_kv * c->head_dim;
      a.pg = pages_view(pool);
      a.rope_table = static_cast<const float*>(m->rope_table.ptr);
      a.rope_layout = c->rope_layout;
      a.span = FA_SPAN;
      a.n_parts = P.fa_parts;
      a.part = P.fa_part;
      a.out_hi = B.att_hi;
      a.out_lo = B.att_lo;
      e = rope_append_rows_launch(a.qkv, a.qkv_stride, B.state, a.rows, a.H, a.Hkv, (int32_t)c->head_dim, a.rope_table,
                                  a.rope_layout, pool->k[l], pool->v[l], c->kv_dtype, a.slot_elems, a.pg, nullptr, nullptr,
                                  s);
      if (e == hipSuccess) e = fattn_launch(a, ctx_end, s);
    } else if (e == hipSuccess) {
      e = launch_batch_kernel(c, m, pool, B, l, BK_ATTN, nullptr, nullptr, nullptr, s);
    }
    mark(PF_ATTN);
    if (e == hipSuccess) {
      PgemmParams g = P.o;
      g.ahi = B.att_hi;
      g.alo = B.att_lo;
      g.w0 = layer_t(m, l, LLMK_WO).ptr;
      g.y = P.y;
      g.out = B.x;
      g.ldo = d;
      e = pgemm_launch(g, PG_RESID, s);
    }
    mark(PF_PROJ);
    if (e == hipSuccess) e = launch_batch_kernel(c, m, pool, B, l, BK_NORM2, nullptr, nullptr, nullptr, s);
    mark(PF_NORM);
    if (e == hipSuccess) {
      PgemmParams g = P.gu;
      g.ahi = B.h_hi;
      g.alo = B.h_lo;
      g.w0 = layer_t(m, l, LLMK_WGATE).ptr;
      g.w1 = layer_t(m, l, LLMK_WUP).ptr;
      g.y = P.y;
      g.uhi = B.u_hi;
      g.ulo = B.u_lo;
      e = pgemm_launch(g, PG_GATEUP, s);
    }
    if (e == hipSuccess) {
      PgemmParams g = P.down;
      g.ahi = B.u_hi;
      g.alo = B.u_lo;
      g.w0 = layer_t(m, l, LLMK_WDOWN).ptr;
      g.y = P.y;
      g.out = B.x;
      g.ldo = d;
      g.hidden = want_hidden ? P.hidden + l * d : nullptr;
      g.hidden_stride = c->n_layer * d;
      e = pgemm_launch(g, PG_RESID, s);
    }
    mark(PF_PROJ);
  }
  if (e == hipSuccess) e = launch_batch_kernel(c, m, pool, B, 0, BK_NORMF, nullptr, nullptr, nullptr, s);
  mark(PF_NORM);
  if (e == hipSuccess) {
    PgemmParams g = P.head;
    g.ahi = B.h_hi;
    g.alo = B.h_lo;
    g.w0 = m->w_out.ptr;
    g.y = P.y;
    e = pgemm_launch(g, PG_NONE, s);
  }
  if (e == hipSuccess)
    e = argmax_launch(P.y, P.head.M, c->vocab, tokens_out, P.am_logit, P.am_val, P.am_idx, P.am_cnt, P.am_bpr, s);
  mark(PF_HEAD);
  if (e == hipSuccess && tm) e = tm->err;
  return e;
}

// Checks of the batched entry points, in the documented order; fills init on success.
int32_t batch_checks(const llmk_config* cfg, const llmk_model* model, const llmk_kv_pool* pool, int64_t B,
                     const int64_t* slots_h, const int64_t* tokens_h, const int64_t* pos_h, int64_t n_steps,
                     const void* out_ptr, const void* ws, BatchInit& init) {
  if (!cfg || !model || !pool || !slots_h || !tokens_h || !pos_h || !out_ptr || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if (B < 1) return LLMK_EMPTY_DIMENSION;
  if (B > LLMK_MAX_BATCH) return LLMK_DIMENSION_TOO_LARGE;
  if ((st = model_check(cfg, model)) != LLMK_OK) return st;
  if ((st = model_lengths(cfg, model)) != LLMK_OK) return st;
  if ((st = pool_check(cfg, pool)) != LLMK_OK) return st;
  if (!weights_aligned(cfg, model) || !batch_config_ok(cfg)) return LLMK_INVALID_ARGUMENT;
  for (int64_t r = 0; r < B; ++r)
    if (slots_h[r] < 0 || slots_h[r] >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  for (int64_t r = 0; r < B; ++r)
    for (int64_t q = 0; q < r; ++q)
      if (slots_h[q] == slots_h[r]) return LLMK_INVALID_ARGUMENT;
  for (int64_t r = 0; r < B; ++r)
    if (tokens_h[r] < 0 || tokens_h[r] >= cfg->vocab) return LLMK_TOKEN_OUT_OF_RANGE;
  for (int64_t r = 0; r < B; ++r)
    if (pos_h[r] < 0 || pos_h[r] + n_steps > cfg->max_seq) return LLMK_POSITION_OUT_OF_RANGE;
  for (int64_t r = 0; r < B; ++r)
    if (pos_h[r] != pool->slot_len_h[slots_h[r]]) return LLMK_CACHE_LENGTH_MISMATCH;
  for (int64_t r = 0; r < B; ++r)
    if (pos_h[r] + n_steps > pool->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  memset(&init, 0, sizeof(init));
  for (int64_t r = 0; r < B; ++r) {
    init.token[r] = (int32_t)tokens_h[r];
    init.pos[r] = (int32_t)pos_h[r];
    init.slot[r] = (int32_t)slots_h[r];
  }
  init.rows = (int32_t)B;
  return LLMK_OK;
}

}  // namespace

// =========================================================================================================
// C ABI
// =========================================================================================================

extern "C" {

const char* llmk_status_name(int32_t code) {
  switch (code) {
    case 560: return "llmk_ok";
    case 561: return "llmk_empty_dimension";
    case 562: return "llmk_a_length_mismatch";
    case 563: return "llmk_b_length_mismatch";
    case 564: return "llmk_dimension_too_large";
    case 565: return "llmk_code_out_of_range";
    case 566: return "llmk_cache_length_mismatch";
    case 567: return "llmk_new_length_mismatch";
    case 568: return "llmk_logits_length_mismatch";
    case 569: return "llmk_gemv_a_length_mismatch";
    case 570: return "llmk_gemv_x_length_mismatch";
    case 571: return "llmk_cache_capacity_exceeded";
    case 572: return "llmk_token_out_of_range";
    case 573: return "llmk_position_out_of_range";
    case 574: return "llmk_head_shape_invalid";
    case 575: return "llmk_slot_out_of_range";
    case 576: return "llmk_weight_length_mismatch";
    case 577: return "llmk_output_length_mismatch";
    case 578: return "llmk_invalid_argument";
    case 579: return "llmk_device_error";
    default: return "llmk_code_out_of_range";
  }
}

int32_t llmk_residual_dims_check(int64_t n, int64_t len_a, int64_t len_b) {
  int32_t st = dims_check({n});
  if (st != LLMK_OK) return st;
  if (len_a != n) return LLMK_A_LENGTH_MISMATCH;
  if (len_b != n) return LLMK_B_LENGTH_MISMATCH;
  return LLMK_OK;
}

int32_t llmk_kv_append_dims_check(int64_t cache_len, int64_t len_cache, int64_t n_new, int64_t len_new) {
  if (cache_len < 0 || n_new < 1) return LLMK_EMPTY_DIMENSION;
  if (cache_len > kMaxDim || n_new > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  if (len_cache != cache_len) return LLMK_CACHE_LENGTH_MISMATCH;
  if (len_new != n_new) return LLMK_NEW_LENGTH_MISMATCH;
  return LLMK_OK;
}

int32_t llmk_argmax_dims_check(int64_t n, int64_t len_logits) {
  int32_t st = dims_check({n});
  if (st != LLMK_OK) return st;
  return len_logits != n ? LLMK_LOGITS_LENGTH_MISMATCH : LLMK_OK;
}

int32_t llmk_gemv_dims_check(int64_t m, int64_t n, int64_t len_a, int64_t len_x) {
  int32_t st = dims_check({m, n});
  if (st != LLMK_OK) return st;
  if (len_a != m * n) return LLMK_GEMV_A_LENGTH_MISMATCH;
  if (len_x != m) return LLMK_GEMV_X_LENGTH_MISMATCH;
  return LLMK_OK;
}

int64_t llmk_gemv_t_workspace_bytes(int64_t m, int64_t n, int32_t a_dtype) {
  if (!is_dtype(a_dtype)) return -LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({m, n});
  if (st != LLMK_OK) return -st;
  return gemv_t_ws_any(m, n, a_dtype);
}

int32_t llmk_gemv_t(const void* a, int64_t len_a, int32_t a_dtype, const float* x, int64_t len_x, int64_t m, int64_t n,
                    float* y, int64_t len_y, void* ws, int64_t len_ws, void* stream) {
  if (!a || !x || !y || !ws || !is_dtype(a_dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = llmk_gemv_dims_check(m, n, len_a, len_x);
  if (st != LLMK_OK) return st;
  if (len_y != n) return LLMK_OUTPUT_LENGTH_MISMATCH;
  GemvT g = plan_gemv_t(m, n, a_dtype, a);
  if (len_ws < gemv_t_ws_any(m, n, a_dtype)) return LLMK_INVALID_ARGUMENT;
  // the vector path needs 16-byte aligned rows; otherwise the scalar path (its own, smaller plan)
  g.p.w0 = a;
  g.p.in = x;
  g.p.in_is_w = 0;
  g.p.y = y;
  if (g.p.ksplit > 1) {
    Carve cv(ws);
    g.p.partial = cv.take<float>((int64_t)g.p.ksplit * g.p.N);
    g.p.counters = cv.take<unsigned>(g.p.n_cblk);
    if (cv.off > len_ws) return LLMK_INVALID_ARGUMENT;
    hipError_t e = fill_u32_launch(g.p.counters, g.p.n_cblk, 0u, as_stream(stream));
    if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  }
  return finish(gemv_launch(g.p, GM_PLAIN, a_dtype == LLMK_BF16, g.vec1, as_stream(stream)));
}

int32_t llmk_gemv(const void* w, int64_t len_w, int32_t w_dtype, const float* x, int64_t len_x, int64_t rows,
                  int64_t cols, float* y, int64_t len_y, void* stream) {
  if (!w || !x || !y || !is_dtype(w_dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, cols});
  if (st != LLMK_OK) return st;
  if (len_w != rows * cols) return LLMK_GEMV_A_LENGTH_MISMATCH;
  if (len_x != cols) return LLMK_GEMV_X_LENGTH_MISMATCH;
  if (len_y != rows) return LLMK_OUTPUT_LENGTH_MISMATCH;
  const int64_t vec = w_dtype == LLMK_BF16 ? 8 : 4;
  if (cols % vec != 0 || !aligned16(w) || cols > 64 * vec * 16)
    return finish(rowdot_simple_launch(w, w_dtype == LLMK_BF16, x, y, rows, cols, as_stream(stream)));
  HeadParams h{};
  h.w = w;
  h.rows = rows;
  h.cols = cols;
  head_plan(h, w_dtype == LLMK_BF16);
  h.x = x;
  h.gain = nullptr;
  h.y = y;
  h.part_val = nullptr;
  return finish(head_launch(h, w_dtype == LLMK_BF16, as_stream(stream)));
}

int32_t llmk_residual_add(const float* a, int64_t len_a, const float* b, int64_t len_b, int64_t n, float* out,
                          int64_t len_out, void* stream) {
  if (!a || !b || !out) return LLMK_INVALID_ARGUMENT;
  int32_t st = llmk_residual_dims_check(n, len_a, len_b);
  if (st != LLMK_OK) return st;
  if (len_out != n) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return finish(residual_add_launch(a, b, out, n, as_stream(stream)));
}

int32_t llmk_add_rmsnorm(float* residual, int64_t len_r, const float* x, int64_t len_x, const float* gain,
                         int64_t len_g, int64_t rows, int64_t n, float eps, float* h, int64_t len_h, void* stream) {
  if (!residual || !gain || !h || !(eps > 0.0f) || !isfinite(eps)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return st;
  if (len_r != rows * n) return LLMK_A_LENGTH_MISMATCH;
  if (x && len_x != rows * n) return LLMK_B_LENGTH_MISMATCH;
  if (len_g != n) return LLMK_WEIGHT_LENGTH_MISMATCH;
  if (len_h != rows * n) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return finish(add_rmsnorm_launch(residual, x, gain, rows, n, eps, h, as_stream(stream)));
}

int32_t llmk_silu_mul(const float* gate, int64_t len_gate, const float* up, int64_t len_up, int64_t n, float* out,
                      int64_t len_out, void* stream) {
  if (!gate || !up || !out) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({n});
  if (st != LLMK_OK) return st;
  if (len_gate != n) return LLMK_A_LENGTH_MISMATCH;
  if (len_up != n) return LLMK_B_LENGTH_MISMATCH;
  if (len_out != n) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return finish(silu_mul_launch(gate, up, out, n, as_stream(stream)));
}

int32_t llmk_rope_table_init(float* table, int64_t len_table, int64_t max_pos, int64_t head_dim, double base,
                             void* stream) {
  if (!table || !(base > 1.0) || !isfinite(base)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({max_pos, head_dim});
  if (st != LLMK_OK) return st;
  if (!rope_head_dim_ok(head_dim)) return LLMK_HEAD_SHAPE_INVALID;
  if (len_table != max_pos * head_dim) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return finish(rope_table_launch(table, max_pos, head_dim, base, as_stream(stream)));
}

int32_t llmk_rope(float* q, int64_t len_q, float* k, int64_t len_k, int64_t rows, int64_t n_q_heads, int64_t n_k_heads,
                  int64_t head_dim, const int32_t* pos, int64_t len_pos, const float* table, int64_t len_table,
                  int64_t max_pos, int32_t layout, void* stream) {
  if (!q || !table || !pos || (layout != LLMK_ROPE_HALF_SPLIT && layout != LLMK_ROPE_INTERLEAVED) ||
      (!k && n_k_heads > 0))
    return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, n_q_heads, head_dim, max_pos});
  if (st != LLMK_OK) return st;
  if (n_k_heads < 0) return LLMK_EMPTY_DIMENSION;
  if (n_k_heads > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  if (!rope_head_dim_ok(head_dim)) return LLMK_HEAD_SHAPE_INVALID;
  if (len_q != rows * n_q_heads * head_dim) return LLMK_A_LENGTH_MISMATCH;
  if (len_k != rows * n_k_heads * head_dim) return LLMK_B_LENGTH_MISMATCH;
  if (len_table != max_pos * head_dim) return LLMK_WEIGHT_LENGTH_MISMATCH;
  if (len_pos != rows) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return finish(rope_launch(q, k, rows, n_q_heads, n_k_heads, head_dim, pos, max_pos, table, layout,
                            as_stream(stream)));
}

int32_t llmk_kv_append_flat(void* cache, int64_t capacity, int32_t dtype, int64_t cache_len, int64_t len_cache,
                            const float* new_vals, int64_t len_new, int64_t n_new, int64_t* new_len_h, void* stream) {
  if (!cache || !new_vals || !is_dtype(dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({capacity});
  if (st != LLMK_OK) return st;
  st = llmk_kv_append_dims_check(cache_len, len_cache, n_new, len_new);
  if (st != LLMK_OK) return st;
  if (cache_len + n_new > capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  st = finish(kv_append_launch(cache, dtype == LLMK_BF16, cache_len, new_vals, n_new, as_stream(stream)));
  if (st == LLMK_OK && new_len_h) *new_len_h = cache_len + n_new;
  return st;
}

int64_t llmk_gqa_attend_workspace_bytes(int64_t ctx_len, int64_t n_head, int64_t head_dim) {
  int32_t st = dims_check({ctx_len, n_head, head_dim});
  if (st != LLMK_OK) return -st;
  Carve c(nullptr);
  c.take<float>(attn_part_floats(n_head, head_dim));
  c.take<unsigned>(n_head);
  return c.off;
}

// the attention launch shared by llmk_gqa_attend_flat and llmk_gqa_attend (every check done)
static int32_t gqa_attend_run(const float* q, const void* k_cache, const void* v_cache, int32_t kv_dtype, int64_t ctx_len,
                              int64_t n_head, int64_t n_kv, int64_t head_dim, float* out, void* ws, void* stream,
                              const KvPaging& pg = KvPaging{}, const float* k_scale = nullptr,
                              const float* v_scale = nullptr) {
  AttnParams a{};
  a.pg = pg;
  a.kv_q8 = kv_dtype == LLMK_Q8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.kv_is_bf16 = kv_dtype == LLMK_BF16;
  a.H = (int32_t)n_head;
  a.Hkv = (int32_t)n_kv;
  a.hd = (int32_t)head_dim;
  a.ctx = (int32_t)ctx_len;
  a.state = nullptr;
  attn_plan(a, ctx_len);
  Carve cv(ws);
  a.part = cv.take<float>(attn_part_floats(n_head, head_dim));
  a.counters = cv.take<unsigned>(n_head);
  a.out = out;
  hipError_t e = fill_u32_launch(a.counters, n_kv, 0u, as_stream(stream));
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  return finish(attn_launch(a, as_stream(stream)));
}

int32_t llmk_gqa_attend_flat(const float* q, int64_t len_q, const void* k_cache, const void* v_cache, int64_t len_cache,
                             int32_t kv_dtype, int64_t ctx_len, int64_t n_head, int64_t n_kv, int64_t head_dim,
                             float* out, int64_t len_out, void* ws, int64_t len_ws, void* stream) {
  if (!q || !k_cache || !v_cache || !out || !ws || !is_dtype(kv_dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({ctx_len, n_head, n_kv, head_dim});
  if (st != LLMK_OK) return st;
  if (n_head % n_kv != 0 || n_head / n_kv > 8 || !attn_head_dim_ok(head_dim)) return LLMK_HEAD_SHAPE_INVALID;
  if (len_q != n_head * head_dim) return LLMK_A_LENGTH_MISMATCH;
  if (len_cache < ctx_len * n_kv * head_dim) return LLMK_B_LENGTH_MISMATCH;
  if (len_out != n_head * head_dim) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (len_ws < llmk_gqa_attend_workspace_bytes(ctx_len, n_head, head_dim)) return LLMK_INVALID_ARGUMENT;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return LLMK_INVALID_ARGUMENT;
  return gqa_attend_run(q, k_cache, v_cache, kv_dtype, ctx_len, n_head, n_kv, head_dim, out, ws, stream);
}

}  // extern "C"

// A pool descriptor's own fields (no config to compare with): 578 / 561 / 564, then the pages.
int32_t llmk::pool_fields_check(const llmk_kv_pool* p) {
  if (!p || !p->k || !p->v || !p->slot_len_h || !is_kv_dtype(p->dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({p->n_layer, p->n_slots, p->capacity, p->n_kv, p->head_dim});
  if (st != LLMK_OK) return st;
  if (p->dtype == LLMK_Q8 && p->head_dim % 16 != 0) return LLMK_HEAD_SHAPE_INVALID;
  for (int64_t l = 0; l < p->n_layer; ++l)
    if (!p->k[l] || !p->v[l] || !aligned16(p->k[l]) || !aligned16(p->v[l])) return LLMK_INVALID_ARGUMENT;
  return p->pages ? pages_check(p) : LLMK_OK;
}

extern "C" {

int32_t llmk_kv_pool_init(llmk_kv_pool* pool) {
  const int32_t st = pool_fields_check(pool);
  if (st != LLMK_OK) return st;
  for (int64_t s = 0; s < pool->n_slots; ++s) pool->slot_len_h[s] = 0;
  for (int64_t i = 0; i < pool->n_layer * pool->n_slots; ++i) {
    if (pool->len_k_h) pool->len_k_h[i] = 0;
    if (pool->len_v_h) pool->len_v_h[i] = 0;
  }
  if (llmk_kv_pages* g = pool->pages) {
    for (int64_t i = 0; i < pool->n_slots * g->max_blocks; ++i) g->table_h[i] = -1;
    for (int64_t b = 0; b < g->n_blocks; ++b) g->refcount_h[b] = 0;
    g->n_free = g->n_blocks;
  }
  return LLMK_OK;
}

int32_t llmk_kv_append(llmk_kv_pool* pool, int64_t layer, int64_t slot, int32_t which, int64_t cache_len,
                       const float* new_vals, int64_t len_new, int64_t n_new, int64_t* new_len_h,
                       int64_t* elem_offset_h, void* stream) {
  if (!new_vals) return LLMK_INVALID_ARGUMENT;
  int32_t st = pool_fields_check(pool);
  if (st != LLMK_OK) return st;
  if (!pool->len_k_h || !pool->len_v_h || (which != 0 && which != 1) || pool->dtype == LLMK_Q8)
    return LLMK_INVALID_ARGUMENT;
  if (layer < 0 || layer >= pool->n_layer) return LLMK_INVALID_ARGUMENT;
  if (cache_len < 0 || n_new < 1) return LLMK_EMPTY_DIMENSION;
  if (cache_len > kMaxDim || n_new > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  int64_t* rec = (which == 0 ? pool->len_k_h : pool->len_v_h) + layer * pool->n_slots + slot;
  if (cache_len != *rec) return LLMK_CACHE_LENGTH_MISMATCH;
  if (len_new != n_new) return LLMK_NEW_LENGTH_MISMATCH;
  const int64_t row = pool->n_kv * pool->head_dim, plane = pool->capacity * row;
  if (cache_len + n_new > plane) return LLMK_CACHE_CAPACITY_EXCEEDED;
  void* buf = which == 0 ? pool->k[layer] : pool->v[layer];
  int64_t off = slot * plane + cache_len;
  if (pool->pages) {
    // the positions the elements fall in, then the elements through the slot's table row
    const int64_t p0 = cache_len / row;
    st = pool_reserve1(pool, slot, p0, (cache_len + n_new + row - 1) / row, as_stream(stream));
    if (st != LLMK_OK) return st;
    off = pages_row(pool, slot, p0) * row + (cache_len - p0 * row);
    st = finish(kv_append_paged_launch(buf, pool->dtype == LLMK_BF16, pages_slot_row(pool, slot), pages_shift(pool),
                                       row, cache_len, new_vals, n_new, as_stream(stream)));
  } else {
    st = finish(kv_append_launch(buf, pool->dtype == LLMK_BF16, off, new_vals, n_new, as_stream(stream)));
  }
  if (st != LLMK_OK) return st;
  *rec = cache_len + n_new;
  if (new_len_h) *new_len_h = *rec;
  if (elem_offset_h) *elem_offset_h = off;
  return LLMK_OK;
}

int32_t llmk_gqa_attend(const float* q, int64_t len_q, const llmk_kv_pool* pool, int64_t layer, int64_t slot,
                        int64_t ctx_len, int64_t n_head, float* out, int64_t len_out, void* ws, int64_t len_ws,
                        void* stream) {
  if (!q || !out || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = pool_fields_check(pool);
  if (st != LLMK_OK) return st;
  if (layer < 0 || layer >= pool->n_layer) return LLMK_INVALID_ARGUMENT;
  st = dims_check({ctx_len, n_head});
  if (st != LLMK_OK) return st;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  const int64_t n_kv = pool->n_kv, hd = pool->head_dim;
  if (n_head % n_kv != 0 || n_head / n_kv > 8 || !attn_head_dim_ok(hd)) return LLMK_HEAD_SHAPE_INVALID;
  if (len_q != n_head * hd) return LLMK_A_LENGTH_MISMATCH;
  if (len_out != n_head * hd) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (ctx_len > pool->capacity) return LLMK_POSITION_OUT_OF_RANGE;
  if (pool->pages)
    for (int64_t p0 = 0; p0 < ctx_len; p0 += pool->pages->block_tokens)
      if (pages_row(pool, slot, p0) < 0) return LLMK_POSITION_OUT_OF_RANGE;
  const int64_t need = ctx_len * n_kv * hd, rec = layer * pool->n_slots + slot;
  if ((pool->len_k_h && pool->len_k_h[rec] < need) || (pool->len_v_h && pool->len_v_h[rec] < need))
    return LLMK_CACHE_LENGTH_MISMATCH;
  if (len_ws < llmk_gqa_attend_workspace_bytes(ctx_len, n_head, hd)) return LLMK_INVALID_ARGUMENT;
  const int64_t esz = dtype_size(pool->dtype), base = pool->pages ? 0 : slot * pool->capacity * n_kv * hd * esz;
  if (base % 16 != 0) return LLMK_INVALID_ARGUMENT;   // the kernel's 16-byte loads need the slot aligned
  KvPaging pg = pages_view(pool);
  pg.table = pages_slot_row(pool, slot);
  const float* ksc = nullptr;
  const float* vsc = nullptr;
  if (pool->dtype == LLMK_Q8) {   // the slot's scales (base / head_dim rows of scales in)
    ksc = pool_scales(pool, pool->k[layer]) + base / hd;
    vsc = pool_scales(pool, pool->v[layer]) + base / hd;
  }
  return gqa_attend_run(q, static_cast<const char*>(pool->k[layer]) + base, static_cast<const char*>(pool->v[layer]) + base,
                        pool->dtype, ctx_len, n_head, n_kv, hd, out, ws, stream, pg, ksc, vsc);
}

int64_t llmk_argmax_workspace_bytes(int64_t rows, int64_t n) {
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return -st;
  const int64_t bpr = n >= 65536 ? 64 : (n + 1023) / 1024;
  Carve c(nullptr);
  c.take<float>(rows * bpr);
  c.take<int32_t>(rows * bpr);
  c.take<unsigned>(rows);
  return c.off;
}

// the argmax launch shared by llmk_argmax and llmk_argmax_noalloc (every check done): partials and tickets
// carved from `ws`, the tickets cleared by a fill kernel
static int32_t argmax_run(const float* logits, int64_t rows, int64_t n, int32_t* token, float* logit, void* ws,
                          void* stream) {
  const int64_t bpr = n >= 65536 ? 64 : (n + 1023) / 1024;
  Carve cv(ws);
  float* pv = cv.take<float>(rows * bpr);
  int32_t* pi = cv.take<int32_t>(rows * bpr);
  unsigned* cnt = cv.take<unsigned>(rows);
  hipError_t e = fill_u32_launch(cnt, rows, 0u, as_stream(stream));
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  return finish(argmax_launch(logits, rows, n, token, logit, pv, pi, cnt, (int32_t)bpr, as_stream(stream)));
}

int32_t llmk_argmax(const float* logits, int64_t len_logits, int64_t rows, int64_t n, int32_t* token, float* logit,
                    void* ws, int64_t len_ws, void* stream) {
  if (!logits || !token || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return st;
  if (len_logits != rows * n) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (len_ws < llmk_argmax_workspace_bytes(rows, n)) return LLMK_INVALID_ARGUMENT;
  if (rows > 65535) return LLMK_DIMENSION_TOO_LARGE;
  return argmax_run(logits, rows, n, token, logit, ws, stream);
}

int32_t llmk_argmax_noalloc(const float* logits, int64_t len_logits, int64_t rows, int64_t n, int32_t* token,
                            float* logit, void* stream) {
  if (!logits || !token) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return st;
  if (len_logits != rows * n) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (rows > LLMK_ARGMAX_NOALLOC_MAX_ROWS || llmk_argmax_workspace_bytes(rows, n) > kArgmaxScratchBytes)
    return LLMK_DIMENSION_TOO_LARGE;
  void* ws = scratch_on(as_stream(stream));
  if (!ws) return LLMK_DEVICE_ERROR;
  return argmax_run(logits, rows, n, token, logit, ws, stream);
}

int64_t llmk_sample_workspace_bytes(int64_t rows, int64_t n, float temperature, int32_t top_k) {
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return -st;
  const int64_t k = temperature == 0.0f ? 1 : (top_k <= 0 || top_k >= n ? n : top_k);
  if (k > LLMK_SAMPLE_MAX_K) return -LLMK_DIMENSION_TOO_LARGE;
  return sample_workspace_bytes(rows, n, (int32_t)k);
}

int32_t llmk_sample(const float* logits, int64_t len_logits, int64_t rows, int64_t n, float temperature,
                    int32_t top_k, float top_p, const float* u, int64_t len_u, int32_t* token, void* ws,
                    int64_t len_ws, void* stream) {
  if (!logits || !u || !token) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, n});
  if (st != LLMK_OK) return st;
  if (len_logits != rows * n) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (len_u != rows) return LLMK_B_LENGTH_MISMATCH;
  if (!(temperature >= 0.0f) || !(top_p > 0.0f && top_p <= 1.0f)) return LLMK_INVALID_ARGUMENT;
  const int64_t k = temperature == 0.0f ? 1 : (top_k <= 0 || top_k >= n ? n : top_k);
  if (k > LLMK_SAMPLE_MAX_K || rows > LLMK_SAMPLE_MAX_ROWS) return LLMK_DIMENSION_TOO_LARGE;
  const int64_t need = sample_workspace_bytes(rows, n, (int32_t)k);
  if (need > 0 && (!ws || len_ws < need || !aligned16(ws))) return LLMK_INVALID_ARGUMENT;
  return finish(sample_launch(logits, rows, n, temperature, (int32_t)k, top_p, u, token, ws, as_stream(stream)));
}

int32_t llmk_kv_slot_offset(const llmk_kv_pool* pool, int64_t slot, int64_t pos, int64_t kv_head, int64_t* offset_h) {
  if (!pool || !offset_h) return LLMK_INVALID_ARGUMENT;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  if (pos < 0 || pos >= pool->capacity) return LLMK_POSITION_OUT_OF_RANGE;
  if (kv_head < 0 || kv_head >= pool->n_kv) return LLMK_HEAD_SHAPE_INVALID;
  const int64_t row = pool->n_kv * pool->head_dim;
  if (pool->pages) {
    if (!pool->pages->table_h || pool->pages->block_tokens < 1) return LLMK_INVALID_ARGUMENT;
    const int64_t r = pages_row(pool, slot, pos);
    if (r < 0) return LLMK_POSITION_OUT_OF_RANGE;
    *offset_h = r * row + kv_head * pool->head_dim;
    return LLMK_OK;
  }
  *offset_h = slot * pool->capacity * row + pos * row + kv_head * pool->head_dim;
  return LLMK_OK;
}

int64_t llmk_decode_workspace_bytes(const llmk_config* cfg, int64_t batch) {
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return -st;
  if (batch < 1) return -LLMK_EMPTY_DIMENSION;
  if (batch > LLMK_MAX_BATCH) return -LLMK_DIMENSION_TOO_LARGE;
  int64_t bytes = 0;
  if (batch == 1) {
    DecodePlan D;
    plan_decode(cfg, nullptr, D);
    bytes = D.bytes;
  } else if (!batch_config_ok(cfg)) {
    return -LLMK_INVALID_ARGUMENT;
  }
  if (batch_config_ok(cfg)) {
    BatchPlan P;
    plan_batch(cfg, batch, nullptr, P);
    bytes = std::max(bytes, P.bytes);
  }
  return bytes;
}

int32_t llmk_decode_step(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                         int64_t token, int64_t pos, float* logits, int64_t len_logits, int32_t* token_out,
                         float* hidden, int64_t len_hidden, void* ws, int64_t len_ws, void* stream) {
  int32_t st = decode_checks(cfg, model, pool, slot, token, pos, 1, token_out, ws);
  if (st != LLMK_OK) return st;
  if (logits && len_logits != cfg->vocab) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (hidden && len_hidden != cfg->n_layer * cfg->d) return LLMK_OUTPUT_LENGTH_MISMATCH;
  DecodePlan D;
  plan_decode(cfg, nullptr, D);
  if (len_ws < D.bytes) return LLMK_INVALID_ARGUMENT;
  plan_decode(cfg, ws, D);
  const int nwg = step_workgroups(cfg);
  if (nwg < 0) return LLMK_INVALID_ARGUMENT;
  hipStream_t s = as_stream(stream);
  if ((st = pool_reserve1(pool, slot, pos, pos + 1, s)) != LLMK_OK) return st;
  hipError_t e;
  if (nwg > 0) {
    e = step_prelude(cfg, model, pool, D, (int32_t)token, (int32_t)pos, s);
    if (e == hipSuccess)
      e = step_launch(step_params(cfg, model, pool, slot, D, nwg, logits, hidden, token_out),
                      cfg->kv_dtype == LLMK_BF16, s);
    // a bounded wait that gave up leaves the error flag set: wait for the step and read it (not possible
    // while the stream is being captured)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (e == hipSuccess) e = hipStreamIsCapturing(s, &cap);
    if (e == hipSuccess && cap == hipStreamCaptureStatusNone) {
      int32_t err = 0;
      e = hipMemcpyAsync(&err, D.step_err, sizeof(err), hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e == hipSuccess && err != 0) return LLMK_DEVICE_ERROR;
    }
  } else {
    e = fill_u32_launch(D.counters, counters_total(cfg, D), 0u, s);
    if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token, (int32_t)pos, s);
    if (e == hipSuccess) e = enqueue_step(cfg, model, pool, slot, D, logits, token_out, hidden, s);
  }
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos + 1);
  return LLMK_OK;
}

// Sampling at the end of every step of the captured loop (null: greedy).
struct LoopSampling {
  float temperature, top_p;
  int32_t k;
  const float* draws;
  void* ws;
};

static int32_t decode_steps_run(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                int64_t token0, int64_t pos0, int64_t n_steps, int32_t* tokens_out, void* ws,
                                int64_t len_ws, void* stream, const LoopSampling* smp);

int32_t llmk_decode_steps(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                          int64_t token0, int64_t pos0, int64_t n_steps, int32_t* tokens_out, int64_t len_tokens,
                          void* ws, int64_t len_ws, void* stream) {
  if (!cfg || !model || !pool || !tokens_out || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if (n_steps < 1) return LLMK_EMPTY_DIMENSION;
  if (n_steps > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  st = decode_checks(cfg, model, pool, slot, token0, pos0, n_steps, tokens_out, ws);
  if (st != LLMK_OK) return st;
  if (len_tokens != n_steps) return LLMK_OUTPUT_LENGTH_MISMATCH;
  return decode_steps_run(cfg, model, pool, slot, token0, pos0, n_steps, tokens_out, ws, len_ws, stream, nullptr);
}

int32_t llmk_decode_steps_sampled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                  int64_t token0, int64_t pos0, int64_t n_steps, float temperature, int32_t top_k,
                                  float top_p, const float* draws, int64_t len_draws, int32_t* tokens_out,
                                  int64_t len_tokens, void* ws, int64_t len_ws, void* sample_ws,
                                  int64_t len_sample_ws, void* stream) {
  if (!cfg || !model || !pool || !tokens_out || !ws || !draws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if (n_steps < 1) return LLMK_EMPTY_DIMENSION;
  if (n_steps > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  st = decode_checks(cfg, model, pool, slot, token0, pos0, n_steps, tokens_out, ws);
  if (st != LLMK_OK) return st;
  if (len_tokens != n_steps) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (len_draws != n_steps) return LLMK_B_LENGTH_MISMATCH;
  if (!(temperature >= 0.0f) || !(top_p > 0.0f && top_p <= 1.0f)) return LLMK_INVALID_ARGUMENT;
  const int64_t n = cfg->vocab;
  const int64_t k = temperature == 0.0f ? 1 : (top_k <= 0 || top_k >= n ? n : top_k);
  if (k > LLMK_SAMPLE_MAX_K) return LLMK_DIMENSION_TOO_LARGE;
  const int64_t need = sample_workspace_bytes(1, n, (int32_t)k);
  if (need > 0 && (!sample_ws || len_sample_ws < need || !aligned16(sample_ws))) return LLMK_INVALID_ARGUMENT;
  const LoopSampling smp{temperature, top_p, (int32_t)k, draws, sample_ws};
  return decode_steps_run(cfg, model, pool, slot, token0, pos0, n_steps, tokens_out, ws, len_ws, stream, &smp);
}

static int32_t decode_steps_run(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                int64_t token0, int64_t pos0, int64_t n_steps, int32_t* tokens_out, void* ws,
                                int64_t len_ws, void* stream, const LoopSampling* smp) {
  DecodePlan D;
  plan_decode(cfg, nullptr, D);
  if (len_ws < D.bytes) return LLMK_INVALID_ARGUMENT;
  plan_decode(cfg, ws, D);
  const int nwg = step_workgroups(cfg);
  if (nwg < 0) return LLMK_INVALID_ARGUMENT;
  hipStream_t s = as_stream(stream);
  // every position the replays write is reserved before the capture
  const int32_t st = pool_reserve1(pool, slot, pos0, pos0 + n_steps, s);
  if (st != LLMK_OK) return st;
  hipError_t e;
  if (nwg > 0) {
    e = step_prelude(cfg, model, pool, D, (int32_t)token0, (int32_t)pos0, s);
  } else {
    e = fill_u32_launch(D.counters, counters_total(cfg, D), 0u, s);
    if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token0, (int32_t)pos0, s);
  }
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;

  // capture one step (token and position come from the device state) and replay it n_steps times
  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    float* lg = smp ? D.logits : nullptr;   // the sampled loop keeps each step's logits for the sampler
    hipError_t ee = nwg > 0 ? step_launch(step_params(cfg, model, pool, slot, D, nwg, lg, nullptr, tokens_out),
                                          cfg->kv_dtype == LLMK_BF16, cs)
                            : enqueue_step(cfg, model, pool, slot, D, lg, tokens_out, nullptr, cs);
    if (smp) {
      // the head advanced the state with its greedy token; the sampled one replaces it
      if (ee == hipSuccess) ee = draw_pick_launch(D.state, smp->draws, D.draw1, cs);
      if (ee == hipSuccess)
        ee = sample_launch(D.logits, 1, cfg->vocab, smp->temperature, smp->k, smp->top_p, D.draw1, D.sampled_tok,
                           smp->ws, cs);
      if (ee == hipSuccess) ee = sampled_token_launch(D.state, D.sampled_tok, tokens_out, cs);
    }
    e = hipStreamEndCapture(cs, &graph);
    if (ee != hipSuccess) e = ee;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  for (int64_t i = 0; e == hipSuccess && i < n_steps; ++i) e = hipGraphLaunch(exec, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  int32_t err = 0;
  if (e == hipSuccess && nwg > 0) e = hipMemcpy(&err, D.step_err, sizeof(err), hipMemcpyDeviceToHost);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (cs) (void)hipStreamDestroy(cs);
  if (e != hipSuccess || err != 0) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos0 + n_steps);
  return LLMK_OK;
}

int32_t llmk_decode_step_batch(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t batch,
                               const int64_t* slots_h, const int64_t* tokens_h, const int64_t* pos_h, float* logits,
                               int64_t len_logits, int32_t* tokens_out, int64_t len_tokens, float* hidden,
                               int64_t len_hidden, void* ws, int64_t len_ws, void* stream) {
  BatchInit init;
  int32_t st = batch_checks(cfg, model, pool, batch, slots_h, tokens_h, pos_h, 1, tokens_out, ws, init);
  if (st != LLMK_OK) return st;
  if (logits && len_logits != batch * cfg->vocab) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (len_tokens != batch) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (hidden && len_hidden != batch * cfg->n_layer * cfg->d) return LLMK_OUTPUT_LENGTH_MISMATCH;
  BatchPlan P;
  plan_batch(cfg, batch, nullptr, P);
  if (len_ws < P.bytes) return LLMK_INVALID_ARGUMENT;
  plan_batch(cfg, batch, ws, P);
  hipStream_t s = as_stream(stream);
  if ((st = batch_reserve(pool, batch, slots_h, pos_h, 1, s)) != LLMK_OK) return st;
  hipError_t e = fill_u32_launch(P.counters, batch_counters_total(cfg, P), 0u, s);
  if (e == hipSuccess) e = set_batch_state_launch(P.state, init, s);
  if (e == hipSuccess) e = enqueue_batch(cfg, model, pool, P, logits, tokens_out, hidden, s);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  for (int64_t r = 0; r < batch; ++r) pool_advance(pool, slots_h[r], pos_h[r] + 1);
  return LLMK_OK;
}

int64_t llmk_prefill_workspace_bytes(const llmk_config* cfg, int64_t n) {
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return -st;
  if (n < 1) return -LLMK_EMPTY_DIMENSION;
  if (n > kMaxDim) return -LLMK_DIMENSION_TOO_LARGE;
  if (!batch_config_ok(cfg)) return -LLMK_INVALID_ARGUMENT;
  return prefill_bytes(cfg, n);
}

}  // extern "C"

namespace {

int32_t prefill_run(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                    const int64_t* tokens_h, int64_t n, int64_t pos0, int32_t* tokens_out, int64_t len_tokens,
                    float* logits, int64_t len_logits, float* hidden, int64_t len_hidden, void* ws, int64_t len_ws,
                    hipStream_t s, PhaseTimer* tm) {
  if (!cfg || !model || !pool || !tokens_h || !tokens_out || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if (n < 1) return LLMK_EMPTY_DIMENSION;
  if (n > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  if ((st = model_check(cfg, model)) != LLMK_OK) return st;
  if ((st = model_lengths(cfg, model)) != LLMK_OK) return st;
  if ((st = pool_check(cfg, pool)) != LLMK_OK) return st;
  if (!weights_aligned(cfg, model) || !batch_config_ok(cfg)) return LLMK_INVALID_ARGUMENT;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  for (int64_t i = 0; i < n; ++i)
    if (tokens_h[i] < 0 || tokens_h[i] >= cfg->vocab) return LLMK_TOKEN_OUT_OF_RANGE;
  if (pos0 < 0 || pos0 + n > cfg->max_seq) return LLMK_POSITION_OUT_OF_RANGE;
  if (pos0 != pool->slot_len_h[slot]) return LLMK_CACHE_LENGTH_MISMATCH;
  if (pos0 + n > pool->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  if (len_tokens != n) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (logits && len_logits != cfg->vocab) return LLMK_LOGITS_LENGTH_MISMATCH;
  if (hidden && len_hidden != cfg->n_layer * cfg->d) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (len_ws < prefill_bytes(cfg, n)) return LLMK_INVALID_ARGUMENT;
  if ((st = pool_reserve1(pool, slot, pos0, pos0 + n, s)) != LLMK_OK) return st;

  hipError_t e = hipSuccess;
  const int64_t rows = std::min(n, kPrefillRows);
  for (int64_t c0 = 0; c0 < n && e == hipSuccess; c0 += rows) {
    // one chunk: prompt rows c0 .. c0 + M - 1 at positions pos0 + c0 + r, all in this slot
    const int64_t M = std::min(rows, n - c0);
    const bool last = c0 + M == n;
    PrefillPlan P;
    plan_prefill(cfg, M, ws, P);
    BatchInit init;
    memset(&init, 0, sizeof(init));
    for (int64_t r = 0; r < M; ++r) {
      init.token[r] = (int32_t)tokens_h[c0 + r];
      init.pos[r] = (int32_t)(pos0 + c0 + r);
      init.slot[r] = (int32_t)slot;
    }
    init.rows = (int32_t)M;
    e = fill_u32_launch(P.rows.counters, batch_counters_total(cfg, P.rows), 0u, s);
    if (e == hipSuccess) e = fill_u32_launch(P.am_cnt, M, 0u, s);
    if (e == hipSuccess) e = set_batch_state_launch(P.rows.state, init, s);
    if (e == hipSuccess) e = enqueue_prefill_chunk(cfg, model, pool, P, pos0 + c0 + M, tokens_out + c0, last && hidden, s, tm);
    if (e == hipSuccess && last && logits)
      e = hipMemcpyAsync(logits, P.y + (M - 1) * cfg->vocab, cfg->vocab * sizeof(float), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && last && hidden)
      e = hipMemcpyAsync(hidden, P.hidden + (M - 1) * cfg->n_layer * cfg->d, cfg->n_layer * cfg->d * sizeof(float),
                         hipMemcpyDeviceToDevice, s);
  }
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos0 + n);
  return LLMK_OK;
}

}  // namespace

extern "C" {

int32_t llmk_prefill(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                     const int64_t* tokens_h, int64_t n, int64_t pos0, int32_t* tokens_out, int64_t len_tokens,
                     float* logits, int64_t len_logits, float* hidden, int64_t len_hidden, void* ws, int64_t len_ws,
                     void* stream) {
  return prefill_run(cfg, model, pool, slot, tokens_h, n, pos0, tokens_out, len_tokens, logits, len_logits, hidden,
                     len_hidden, ws, len_ws, as_stream(stream), nullptr);
}

int32_t llmk_prefill_profiled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                              const int64_t* tokens_h, int64_t n, int64_t pos0, int32_t* tokens_out,
                              int64_t len_tokens, float* class_ms_h, int64_t len_class_ms, void* ws, int64_t len_ws,
                              void* stream) {
  if (!class_ms_h) return LLMK_INVALID_ARGUMENT;
  if (len_class_ms < PF_CLASSES) return LLMK_OUTPUT_LENGTH_MISMATCH;
  PhaseTimer tm;
  tm.s = as_stream(stream);
  int32_t st = prefill_run(cfg, model, pool, slot, tokens_h, n, pos0, tokens_out, len_tokens, nullptr, 0, nullptr, 0,
                           ws, len_ws, tm.s, &tm);
  if (st != LLMK_OK) return st;
  hipError_t e = hipStreamSynchronize(tm.s);
  for (int k = 0; k < PF_CLASSES; ++k) class_ms_h[k] = 0.0f;
  for (size_t i = 1; e == hipSuccess && i < tm.ev.size(); ++i) {
    if (tm.cls[i] < 0) continue;
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, tm.ev[i - 1], tm.ev[i]);
    class_ms_h[tm.cls[i]] += ms;
  }
  return e == hipSuccess ? LLMK_OK : LLMK_DEVICE_ERROR;
}

int32_t llmk_decode_steps_batch(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t batch,
                                const int64_t* slots_h, const int64_t* tokens0_h, const int64_t* pos0_h,
                                int64_t n_steps, int32_t* tokens_out, int64_t len_tokens, void* ws, int64_t len_ws,
                                void* stream) {
  if (!cfg || !model || !pool || !slots_h || !tokens0_h || !pos0_h || !tokens_out || !ws) return LLMK_INVALID_ARGUMENT;
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  if (n_steps < 1) return LLMK_EMPTY_DIMENSION;
  if (n_steps > kMaxDim) return LLMK_DIMENSION_TOO_LARGE;
  BatchInit init;
  st = batch_checks(cfg, model, pool, batch, slots_h, tokens0_h, pos0_h, n_steps, tokens_out, ws, init);
  if (st != LLMK_OK) return st;
  if (len_tokens != n_steps * batch) return LLMK_OUTPUT_LENGTH_MISMATCH;
  BatchPlan P;
  plan_batch(cfg, batch, nullptr, P);
  if (len_ws < P.bytes) return LLMK_INVALID_ARGUMENT;
  plan_batch(cfg, batch, ws, P);
  hipStream_t s = as_stream(stream);
  if ((st = batch_reserve(pool, batch, slots_h, pos0_h, n_steps, s)) != LLMK_OK) return st;
  hipError_t e = fill_u32_launch(P.counters, batch_counters_total(cfg, P), 0u, s);
  if (e == hipSuccess) e = set_batch_state_launch(P.state, init, s);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;

  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t ee = enqueue_batch(cfg, model, pool, P, nullptr, tokens_out, nullptr, cs);
    e = hipStreamEndCapture(cs, &graph);
    if (ee != hipSuccess) e = ee;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  for (int64_t i = 0; e == hipSuccess && i < n_steps; ++i) e = hipGraphLaunch(exec, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (cs) (void)hipStreamDestroy(cs);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  for (int64_t r = 0; r < batch; ++r) pool_advance(pool, slots_h[r], pos0_h[r] + n_steps);
  return LLMK_OK;
}

int64_t llmk_decode_kernel_count(const llmk_config* cfg) {
  int32_t st = config_check(cfg);
  if (st != LLMK_OK) return -st;
  return 5 * cfg->n_layer + 1;
}

int32_t llmk_decode_step_profiled(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                  int64_t token, int64_t pos, int32_t* token_out, float* kernel_ms_h,
                                  int64_t len_kernel_ms, void* ws, int64_t len_ws, void* stream) {
  if (!kernel_ms_h) return LLMK_INVALID_ARGUMENT;
  int32_t st = decode_checks(cfg, model, pool, slot, token, pos, 1, token_out, ws);
  if (st != LLMK_OK) return st;
  const int64_t nk = 5 * cfg->n_layer + 1;
  if (len_kernel_ms < nk) return LLMK_OUTPUT_LENGTH_MISMATCH;
  DecodePlan D;
  plan_decode(cfg, nullptr, D);
  if (len_ws < D.bytes) return LLMK_INVALID_ARGUMENT;
  plan_decode(cfg, ws, D);
  hipStream_t s = as_stream(stream);
  if ((st = pool_reserve1(pool, slot, pos, pos + 1, s)) != LLMK_OK) return st;
  hipEvent_t* ev = new hipEvent_t[2 * nk]();
  hipError_t e = hipSuccess;
  int64_t made = 0;
  for (; made < 2 * nk && e == hipSuccess; ++made) e = hipEventCreate(&ev[made]);
  if (e == hipSuccess) e = fill_u32_launch(D.counters, counters_total(cfg, D), 0u, s);
  if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token, (int32_t)pos, s);
  if (e == hipSuccess) e = enqueue_step(cfg, model, pool, slot, D, nullptr, token_out, nullptr, s, ev);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  for (int64_t k = 0; e == hipSuccess && k < nk; ++k) e = hipEventElapsedTime(&kernel_ms_h[k], ev[2 * k], ev[2 * k + 1]);
  for (int64_t i = 0; i < made; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  delete[] ev;
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos + 1);
  return LLMK_OK;
}

int32_t llmk_decode_path(const llmk_config* cfg) {
  if (!cfg) return LLMK_INVALID_ARGUMENT;
  const int32_t st = config_check(cfg);
  if (st != LLMK_OK) return st;
  const int nwg = step_workgroups(cfg);
  if (nwg < 0) return LLMK_INVALID_ARGUMENT;
  return nwg > 0 ? LLMK_STEP_PERSISTENT : LLMK_STEP_PER_OP;
}

int32_t llmk_decode_kernel_time(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool, int64_t slot,
                                int64_t token, int64_t pos, int32_t kernel, int32_t reps, int32_t* token_out,
                                float* ms_per_launch_h, void* ws, int64_t len_ws, void* stream) {
  if (!ms_per_launch_h) return LLMK_INVALID_ARGUMENT;
  int32_t st = decode_checks(cfg, model, pool, slot, token, pos, 1, token_out, ws);
  if (st != LLMK_OK) return st;
  if (kernel < 0 || kernel > K_STEP) return LLMK_INVALID_ARGUMENT;
  if (reps < 1) return LLMK_EMPTY_DIMENSION;
  if (reps > kTimeMaxReps) return LLMK_DIMENSION_TOO_LARGE;
  DecodePlan D;
  plan_decode(cfg, nullptr, D);
  if (len_ws < D.bytes) return LLMK_INVALID_ARGUMENT;
  plan_decode(cfg, ws, D);
  hipStream_t s = as_stream(stream);
  if (kernel == K_STEP && pos + reps > pool->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  if ((st = pool_reserve1(pool, slot, pos, pos + (kernel == K_STEP ? reps : 1), s)) != LLMK_OK) return st;
  if (kernel == K_STEP) return time_step_kernel(cfg, model, pool, slot, token, pos, reps, token_out, ms_per_launch_h, D, s);
  // one ordinary step leaves valid activations in the workspace; the state is then reset to (token, pos)
  // so that repeated attention launches stay at pos
  hipError_t e = fill_u32_launch(D.counters, counters_total(cfg, D), 0u, s);
  if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token, (int32_t)pos, s);
  if (e == hipSuccess) e = enqueue_step(cfg, model, pool, slot, D, nullptr, token_out, nullptr, s);
  if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token, (int32_t)pos, s);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;

  // the class's launches (every layer, reps times) captured back to back into one graph, replayed once
  // between two events on the caller's stream
  const int64_t per_rep = kernel == K_HEAD ? 1 : cfg->n_layer;
  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t ee = hipSuccess;
    for (int32_t r = 0; r < reps && ee == hipSuccess; ++r)
      for (int64_t l = 0; l < per_rep && ee == hipSuccess; ++l)
        ee = launch_kernel(cfg, model, pool, slot, D, l, kernel, nullptr, D.tok_scratch, nullptr, cs);
    e = hipStreamEndCapture(cs, &graph);
    if (ee != hipSuccess) e = ee;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = hipGraphLaunch(exec, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  // the repeated launches scrambled the workspace and (attention) the K/V at pos of every layer: one more
  // ordinary step puts back exactly what llmk_decode_step leaves
  if (e == hipSuccess) e = set_state_launch(D.state, (int32_t)token, (int32_t)pos, s);
  if (e == hipSuccess) e = enqueue_step(cfg, model, pool, slot, D, nullptr, token_out, nullptr, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (cs) (void)hipStreamDestroy(cs);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  pool_advance(pool, slot, pos + 1);
  *ms_per_launch_h = ms / (float)(reps * per_rep);
  return LLMK_OK;
}

int32_t llmk_decode_batch_kernel_time(const llmk_config* cfg, const llmk_model* model, llmk_kv_pool* pool,
                                      int64_t batch, const int64_t* slots_h, const int64_t* tokens_h,
                                      const int64_t* pos_h, int32_t kernel, int32_t reps, int32_t* tokens_out,
                                      float* ms_per_launch_h, void* ws, int64_t len_ws, void* stream) {
  if (!ms_per_launch_h) return LLMK_INVALID_ARGUMENT;
  BatchInit init;
  int32_t st = batch_checks(cfg, model, pool, batch, slots_h, tokens_h, pos_h, 1, tokens_out, ws, init);
  if (st != LLMK_OK) return st;
  if (kernel < 0 || kernel >= BK_CLASSES) return LLMK_INVALID_ARGUMENT;
  if (reps < 1) return LLMK_EMPTY_DIMENSION;
  if (reps > kTimeMaxReps) return LLMK_DIMENSION_TOO_LARGE;
  BatchPlan P;
  plan_batch(cfg, batch, nullptr, P);
  if (len_ws < P.bytes) return LLMK_INVALID_ARGUMENT;
  plan_batch(cfg, batch, ws, P);
  hipStream_t s = as_stream(stream);
  if ((st = batch_reserve(pool, batch, slots_h, pos_h, 1, s)) != LLMK_OK) return st;
  // one ordinary step leaves valid activations; the state is reset so repeated attention stays at pos
  hipError_t e = fill_u32_launch(P.counters, batch_counters_total(cfg, P), 0u, s);
  if (e == hipSuccess) e = set_batch_state_launch(P.state, init, s);
  if (e == hipSuccess) e = enqueue_batch(cfg, model, pool, P, nullptr, tokens_out, nullptr, s);
  if (e == hipSuccess) e = set_batch_state_launch(P.state, init, s);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;

  const int64_t per_rep = (kernel == BK_NORMF || kernel == BK_HEAD) ? 1 : cfg->n_layer;
  hipStream_t cs = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    hipError_t ee = hipSuccess;
    for (int32_t r = 0; r < reps && ee == hipSuccess; ++r)
      for (int64_t l = 0; l < per_rep && ee == hipSuccess; ++l)
        ee = launch_batch_kernel(cfg, model, pool, P, l, kernel, nullptr, P.tok_scratch, nullptr, cs);
    e = hipStreamEndCapture(cs, &graph);
    if (ee != hipSuccess) e = ee;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = hipGraphLaunch(exec, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  // one more ordinary step rewrites what the repeated launches disturbed
  if (e == hipSuccess) e = set_batch_state_launch(P.state, init, s);
  if (e == hipSuccess) e = enqueue_batch(cfg, model, pool, P, nullptr, tokens_out, nullptr, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (cs) (void)hipStreamDestroy(cs);
  if (e != hipSuccess) return LLMK_DEVICE_ERROR;
  for (int64_t r = 0; r < batch; ++r) pool_advance(pool, slots_h[r], pos_h[r] + 1);
  *ms_per_launch_h = ms / (float)(reps * per_rep);
  return LLMK_OK;
}

int64_t llmk_q8_pack_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim || cols % Q8_GROUP != 0) return -1;
  return q8_pack_bytes(rows, cols);
}

int32_t llmk_quantize_q8(const void* w, int64_t len_w, int32_t w_dtype, int64_t rows, int64_t cols, void* pack,
                         int64_t len_pack, void* stream) {
  if (!w || !pack || !is_dtype(w_dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, cols});
  if (st != LLMK_OK) return st;
  if (cols % Q8_GROUP != 0) return LLMK_HEAD_SHAPE_INVALID;
  if (len_w != rows * cols) return LLMK_WEIGHT_LENGTH_MISMATCH;
  if (len_pack != q8_pack_bytes(rows, cols)) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (!aligned16(w) || !aligned16(pack)) return LLMK_INVALID_ARGUMENT;
  return finish(q8_quantize_launch(w, w_dtype == LLMK_BF16, rows, cols, pack, as_stream(stream)));
}

int32_t llmk_transpose(const void* src, int64_t len_src, void* dst, int64_t len_dst, int64_t rows, int64_t cols,
                       int32_t dtype, void* stream) {
  if (!src || !dst || !is_dtype(dtype)) return LLMK_INVALID_ARGUMENT;
  int32_t st = dims_check({rows, cols});
  if (st != LLMK_OK) return st;
  if (len_src != rows * cols) return LLMK_A_LENGTH_MISMATCH;
  if (len_dst != rows * cols) return LLMK_OUTPUT_LENGTH_MISMATCH;
  if (src == dst) return LLMK_INVALID_ARGUMENT;
  return finish(transpose_launch(src, dst, rows, cols, dtype == LLMK_BF16, as_stream(stream)));
}

}  // extern "C"
