// The whole decode step of one sequence as one persistent kernel (gfx950).
//
// A step is a chain of operations each of which needs all of the previous one's output: RMSNorm + q|k|v,
// attention, o + residual, RMSNorm + gate|up, down + residual, per layer, then the head and the greedy
// token ("The forward pass end to end", "What a forward step does"). As separate kernels each operation
// pays a launch, a ramp-up and a drain, about as long as a small projection itself. Here one workgroup per
// CU runs the whole step: the operations are separated by grid barriers, and every workgroup streams its
// share of the weights through a ring of 16-byte loads per lane that runs one group of SK_RING loads ahead
// of the arithmetic, across the barriers, so the next operation's first weights are already on chip when
// its input becomes available ("Inside the engine", "4. The pipelined decode": keep the device busy
// between the step's pieces).
//
// Work split. Every projection y = W v is cut into equal row slices, one per workgroup; inside a
// workgroup the 8 waves split K, lane l of wave w reads 8 consecutive bf16 of a row per load (16 B), and
// the waves' partial sums meet in LDS. The input vector v (normalised x, the attention output or u) is
// staged in LDS by every workgroup. The head is cut the same way into chunks of at most SK_ROWS rows.
// Attention items (K/V head, context part) are spread over the workgroups as in the attention kernel.
//
// Coherence. Activations written in this launch by one workgroup and read by another go through
// device-scope stores and loads (each XCD's L2 is not coherent with the others); weights and the K/V
// history are only read, so they use ordinary loads. A barrier is: every thread waits for its own stores,
// one thread adds 1 to a 64-bit arrival counter and spins (with sleep) until all workgroups of this
// barrier have arrived. The spin is bounded; a workgroup that gives up sets an error flag and leaves,
// the others then time out too, and the host reports a device error rather than hanging.
#include <limits.h>

#include "attn_block.h"

namespace llmk {

constexpr int SK_THREADS = ATTN_THREADS;   // 512: 8 waves
constexpr int SK_WAVES = SK_THREADS / 64;
constexpr int SK_RING = 16;                 // weight loads per lane per group; the ring holds one group
constexpr int SK_ROWS = 128;                // rows per phase chunk per workgroup
constexpr int SK_SEG = 512;                 // elements one wave covers per load (64 lanes x 8)
constexpr int SK_MAX_LAYERS = STEP_MAX_LAYERS;   // layer table held in LDS
constexpr unsigned SK_SPIN_LIMIT = 1u << 20;   // about a second of waiting

enum { PK_QKV = 0, PK_O = 1, PK_GU = 2, PK_DN = 3, PK_HEAD = 4 };

// One phase: a chunk of this workgroup's rows of one operation. Its units are (row r, load i) with
// i < 2^sh (the loads per row rounded up to a power of two), in the order u = r * 2^sh + i, padded to
// whole groups of SK_RING units. GATEUP chunks order their rows gate first, then up.
struct Phase {
  int kind, l, chunk;
  int R;                // rows (GATEUP: 2 per output)
  int row0;             // first global row (GATEUP: first output)
  int K, KS;            // row length, elements per wave
  int sh;               // log2 of the loads per row
  int groups;           // SK_RING-unit groups (0 when R == 0)
};

__device__ __forceinline__ int sk_cdiv(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int sk_clamp0(int v, int hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

struct Split { int rq, ro, rg, rd, rh; int cq, co, cg, cd, ch; int per_layer; };

__device__ __forceinline__ Split sk_split(const StepParams& p) {
  Split s;
  s.rq = sk_cdiv(p.qd + 2 * p.kvd, p.nwg);
  s.ro = sk_cdiv(p.d, p.nwg);
  s.rg = sk_cdiv(p.F, p.nwg);             // outputs; rows = 2 per output
  s.rd = sk_cdiv(p.d, p.nwg);
  s.rh = sk_cdiv(p.V, p.nwg);
  s.cq = sk_cdiv(s.rq, SK_ROWS);
  s.co = sk_cdiv(s.ro, SK_ROWS);
  s.cg = sk_cdiv(s.rg, SK_ROWS / 2);
  s.cd = sk_cdiv(s.rd, SK_ROWS);
  s.ch = sk_cdiv(s.rh, SK_ROWS);
  s.per_layer = s.cq + s.co + s.cg + s.cd;
  return s;
}

__device__ __forceinline__ int sk_n_phases(const StepParams& p, const Split& s) { return p.n_layer * s.per_layer + s.ch; }

__device__ __forceinline__ Phase sk_phase(const StepParams& p, const Split& s, int ph, int w) {
  Phase f;
  int kind, l, c;
  if (ph < p.n_layer * s.per_layer) {
    l = ph / s.per_layer;
    c = ph % s.per_layer;
    if (c < s.cq) { kind = PK_QKV; }
    else if ((c -= s.cq) < s.co) { kind = PK_O; }
    else if ((c -= s.co) < s.cg) { kind = PK_GU; }
    else { c -= s.cg; kind = PK_DN; }
  } else {
    kind = PK_HEAD;
    l = 0;
    c = ph - p.n_layer * s.per_layer;
  }
  f.kind = kind;
  f.l = l;
  f.chunk = c;
  int n_rows, per;   // global rows (outputs) of the operation, rows (outputs) per workgroup
  switch (kind) {
    case PK_QKV: n_rows = p.qd + 2 * p.kvd; per = s.rq; f.K = p.d; break;
    case PK_O: n_rows = p.d; per = s.ro; f.K = p.qd; break;
    case PK_GU: n_rows = p.F; per = s.rg; f.K = p.d; break;
    case PK_DN: n_rows = p.d; per = s.rd; f.K = p.F; break;
    default: n_rows = p.V; per = s.rh; f.K = p.d; break;
  }
  const int step = kind == PK_GU ? SK_ROWS / 2 : SK_ROWS;
  const int mine = sk_clamp0(n_rows - w * per, per);
  const int in_chunk = sk_clamp0(mine - c * step, step);
  f.row0 = w * per + c * step;
  f.R = kind == PK_GU ? 2 * in_chunk : in_chunk;
  f.KS = (sk_cdiv(f.K, SK_WAVES) + 7) / 8 * 8;
  const int ni = sk_cdiv(f.KS, SK_SEG);
  f.sh = 0;
  while ((1 << f.sh) < ni) ++f.sh;
  f.groups = sk_cdiv(f.R << f.sh, SK_RING);
  return f;
}

// the weight row behind local row r of phase f (layer table in LDS; no global memory access)
__device__ __forceinline__ const bf16_t* sk_row(const StepParams& p, const StepLayer* lt, const Phase& f, int r) {
  if (f.kind == PK_HEAD) return p.w_out + (int64_t)(f.row0 + r) * p.d;
  const StepLayer& L = lt[f.l];
  switch (f.kind) {
    case PK_QKV: {
      const int gr = f.row0 + r;
      if (gr < p.qd) return L.w[0] + (int64_t)gr * p.d;
      if (gr < p.qd + p.kvd) return L.w[1] + (int64_t)(gr - p.qd) * p.d;
      return L.w[2] + (int64_t)(gr - p.qd - p.kvd) * p.d;
    }
    case PK_GU: {
      const int half = f.R >> 1;
      return (r < half ? L.w[4] + (int64_t)(f.row0 + r) * p.d : L.w[5] + (int64_t)(f.row0 + r - half) * p.d);
    }
    case PK_O: return L.w[3] + (int64_t)(f.row0 + r) * p.qd;
    default: return L.w[6] + (int64_t)(f.row0 + r) * p.F;
  }
}

// grid barrier (see the header comment); returns false after a timeout
__device__ __forceinline__ bool sk_barrier(const StepParams& p, unsigned long long target, int* s_ok) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(p.bar, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned n = 0;
    int ok = 1;
    while (__hip_atomic_load(p.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++n > SK_SPIN_LIMIT || ld_dev(p.err) != 0) {
        ok = 0;
        st_dev(p.err, 1);
        break;
      }
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// vin[0..n) = x * rsqrt(mean(x^2) + eps) * g. x is a buffer version written earlier in this launch and
// never read before it in this launch, so no L2 holds a stale copy and ordinary loads see the data.
__device__ __forceinline__ void sk_stage_norm(const float* x, const float* g, int n, float eps, float* vin,
                                              float* s_red) {
  float ss = 0.0f;
  for (int i = threadIdx.x * 4; i < n; i += SK_THREADS * 4) {
    const float4 v = *reinterpret_cast<const float4*>(x + i);
    *reinterpret_cast<float4*>(vin + i) = v;
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
  }
  ss = wave_sum_dpp(ss);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < SK_WAVES; ++w) tot += s_red[w];
  const float scale = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += SK_THREADS) vin[i] = vin[i] * scale * g[i];
  __syncthreads();
}

// vin[0..n) = src (a buffer version, as above)
__device__ __forceinline__ void sk_stage_copy(const float* src, int n, float* vin) {
  for (int i = threadIdx.x * 4; i < n; i += SK_THREADS * 4)
    *reinterpret_cast<float4*>(vin + i) = *reinterpret_cast<const float4*>(src + i);
  __syncthreads();
}

template <typename T, int HD>
__global__ __launch_bounds__(SK_THREADS) void step_kernel(const StepParams p) {
  extern __shared__ float vin[];                         // the phase's input vector (max(d, qd, F) floats)
  __shared__ float s_part[SK_ROWS][SK_WAVES + 1];         // per-row partial sums of the 8 waves
  __shared__ StepLayer s_layers[SK_MAX_LAYERS];
  __shared__ float s_red[SK_WAVES];
  __shared__ float s_best_v[SK_WAVES];
  __shared__ int s_best_i[SK_WAVES];
  __shared__ int s_ok;
  __shared__ int s_last;

  const int w = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Split sp = sk_split(p);
  const int n_ph = sk_n_phases(p, sp);
  const int step = p.state->step;
  const int nb_step = 5 * p.n_layer + 1;                 // barriers per step
  unsigned long long bar_idx = (unsigned long long)step * nb_step;   // barriers passed so far in this call
  const unsigned long long nwg = (unsigned long long)p.nwg;

  // the layer table in LDS: weight addresses are then computed without global loads (which would make the
  // ring's loads wait), and every workgroup reads it once
  for (int i = threadIdx.x; i < p.n_layer; i += SK_THREADS) s_layers[i] = p.layers[i];
  __syncthreads();

  // activation buffer versions: x_v (v = 0 embedding, 2l+1 after layer l's o, 2l+2 after its down), and
  // per layer q|k|v, attention output and u
#define LLMK_SK_X(V) (p.x + (int64_t)(V) * p.x_stride)
#define LLMK_SK_QKV(L) (p.qkv + (int64_t)(L) * p.qkv_stride)
#define LLMK_SK_ATT(L) (p.att + (int64_t)(L) * p.att_stride)
#define LLMK_SK_U(L) (p.u + (int64_t)(L) * p.u_stride)

  AttnParams ap{};
  ap.H = p.H;
  ap.Hkv = p.Hkv;
  ap.hd = HD;
  ap.kv_is_bf16 = sizeof(T) == 2;
  ap.state = p.state;
  ap.chunk = p.attn_chunk;
  ap.sub_per_wg = p.attn_sub_per_wg;
  ap.n_parts = p.attn_n_parts;
  ap.part = p.attn_part;
  ap.counters = p.attn_cnt;
  ap.rope_table = p.rope_table;
  ap.rope_layout = p.rope_layout;

  // x_0 = emb[token]: each workgroup writes a slice
  {
    const int tok = p.state->token;
    const int per = sk_cdiv(p.d, p.nwg);
    for (int i = w * per + threadIdx.x; i < min(p.d, (w + 1) * per); i += SK_THREADS)
      st_dev(LLMK_SK_X(0) + i, bf16_to_f32(p.emb[(int64_t)tok * p.d + i]));
  }

  // ---- the feed: which group of which phase the ring loads next ----
  int fph = 0, fg = 0;
  Phase ff = sk_phase(p, sp, 0, w);
  while (fph < n_ph && ff.groups == 0) {
    if (++fph < n_ph) ff = sk_phase(p, sp, fph, w);
  }
  uint4 ring[SK_RING];
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  // load j of the feed's current group; lanes with nothing to read load from w_out and hold zero, so every
  // lane issues every load (straight-line code whose completion the compiler counts)
#define LLMK_SK_FEED(J)                                                                       \
  {                                                                                           \
    const int u_ = fg * SK_RING + (J);                                                        \
    const int r_ = u_ >> ff.sh, i_ = u_ & ((1 << ff.sh) - 1);                                 \
    const int k_ = wave * ff.KS + i_ * SK_SEG + lane * 8;                                     \
    const bool ok_ = fph < n_ph && r_ < ff.R && k_ < min((wave + 1) * ff.KS, ff.K);            \
    const bf16_t* a_ = ok_ ? sk_row(p, s_layers, ff, r_) + k_ : p.w_out;                      \
    const uint4 v_ = *reinterpret_cast<const uint4*>(a_);                                     \
    ring[J] = ok_ ? v_ : zero;                                                                \
  }
#define LLMK_SK_FEED_NEXT()                                                                   \
  if (fph < n_ph && ++fg == ff.groups) {                                                      \
    fg = 0;                                                                                   \
    do {                                                                                      \
      if (++fph < n_ph) ff = sk_phase(p, sp, fph, w);                                         \
    } while (fph < n_ph && ff.groups == 0);                                                   \
  }
#pragma unroll
  for (int j = 0; j < SK_RING; ++j) LLMK_SK_FEED(j)
  LLMK_SK_FEED_NEXT()

  float best_v = -INFINITY;   // head: this workgroup's best logit so far (thread 0)
  int best_i = INT_MAX;

  for (int ph = 0; ph < n_ph; ++ph) {
    const Phase f = sk_phase(p, sp, ph, w);
    // ---- input of the phase ----
    if (f.chunk == 0) {
      if (f.kind == PK_O) {
        if (!sk_barrier(p, ++bar_idx * nwg, &s_ok)) return;
        // RoPE, K/V append and attention of layer l (this workgroup's items), merged output in att_l
        const StepLayer& L = s_layers[f.l];
        ap.qkv_raw = LLMK_SK_QKV(f.l);
        ap.out = LLMK_SK_ATT(f.l);
        ap.k = static_cast<const char*>(L.k) + p.kv_off * (int64_t)sizeof(T);
        ap.v = static_cast<const char*>(L.v) + p.kv_off * (int64_t)sizeof(T);
        ap.k_w = static_cast<char*>(L.k) + p.kv_off * (int64_t)sizeof(T);
        ap.v_w = static_cast<char*>(L.v) + p.kv_off * (int64_t)sizeof(T);
        for (int it = w; it < p.Hkv * p.attn_n_parts; it += p.nwg)
          attn_block<T, HD>(ap, it / p.attn_n_parts, it % p.attn_n_parts, 0);
      }
      if (!sk_barrier(p, ++bar_idx * nwg, &s_ok)) return;
      switch (f.kind) {
        case PK_QKV: sk_stage_norm(LLMK_SK_X(2 * f.l), s_layers[f.l].g1, p.d, p.eps, vin, s_red); break;
        case PK_O: sk_stage_copy(LLMK_SK_ATT(f.l), p.qd, vin); break;
        case PK_GU: sk_stage_norm(LLMK_SK_X(2 * f.l + 1), s_layers[f.l].g2, p.d, p.eps, vin, s_red); break;
        case PK_DN: sk_stage_copy(LLMK_SK_U(f.l), p.F, vin); break;
        default: sk_stage_norm(LLMK_SK_X(2 * p.n_layer), p.g_final, p.d, p.eps, vin, s_red); break;
      }
    }
    // ---- the phase's groups: row dots from the ring while the ring is refilled with the feed's next group
    float acc = 0.0f;
    const int lastld = (1 << f.sh) - 1;
    for (int g = 0; g < f.groups; ++g) {
#pragma unroll
      for (int j = 0; j < SK_RING; ++j) {
        const int u = g * SK_RING + j;
        const int r = u >> f.sh, i = u & lastld;
        // lanes with nothing to read hold zero in the ring; they read a clamped, valid part of vin
        const int k = min(wave * f.KS + i * SK_SEG + lane * 8, f.K - 8);
        const float4 v0 = *reinterpret_cast<const float4*>(vin + k);
        const float4 v1 = *reinterpret_cast<const float4*>(vin + k + 4);
        float wf[8];
        unpack<bf16_t, 8>(ring[j], wf);
        acc = fmaf(wf[0], v0.x, acc);
        acc = fmaf(wf[1], v0.y, acc);
        acc = fmaf(wf[2], v0.z, acc);
        acc = fmaf(wf[3], v0.w, acc);
        acc = fmaf(wf[4], v1.x, acc);
        acc = fmaf(wf[5], v1.y, acc);
        acc = fmaf(wf[6], v1.z, acc);
        acc = fmaf(wf[7], v1.w, acc);
        if (i == lastld) {
          if (r < f.R) {
            const float s = wave_sum_dpp(acc);
            if (lane == 0) s_part[r][wave] = s;
          }
          acc = 0.0f;
        }
        LLMK_SK_FEED(j)
      }
      LLMK_SK_FEED_NEXT()
    }
    __syncthreads();
    // ---- epilogue: the rows' sums over the waves, in wave order ----
    const int t = threadIdx.x;
    switch (f.kind) {
      case PK_QKV:
        if (t < f.R) {
          float y = 0.0f;
#pragma unroll
          for (int q = 0; q < SK_WAVES; ++q) y += s_part[t][q];
          st_dev(LLMK_SK_QKV(f.l) + f.row0 + t, y);
        }
        break;
      case PK_O:
      case PK_DN:
        if (t < f.R) {
          float y = 0.0f;
#pragma unroll
          for (int q = 0; q < SK_WAVES; ++q) y += s_part[t][q];
          const int n = f.row0 + t;
          const int v = 2 * f.l + (f.kind == PK_O ? 0 : 1);   // x_v + y -> x_{v+1}
          const float xn = LLMK_SK_X(v)[n] + y;
          st_dev(LLMK_SK_X(v + 1) + n, xn);
          if (f.kind == PK_DN && p.hidden) p.hidden[(int64_t)f.l * p.d + n] = xn;
        }
        break;
      case PK_GU:
        if (t < f.R / 2) {
          float g = 0.0f, up = 0.0f;
#pragma unroll
          for (int q = 0; q < SK_WAVES; ++q) {
            g += s_part[t][q];
            up += s_part[t + f.R / 2][q];
          }
          st_dev(LLMK_SK_U(f.l) + f.row0 + t, silu_f(g) * up);
        }
        break;
      default: {   // head: logits and this chunk's best, folded into the workgroup's best
        float v = -INFINITY;
        int ix = INT_MAX;
        if (t < f.R) {
          float y = 0.0f;
#pragma unroll
          for (int q = 0; q < SK_WAVES; ++q) y += s_part[t][q];
          v = y;
          ix = f.row0 + t;
          if (p.logits) p.logits[ix] = y;
        }
        wave_argmax(v, ix);
        if (lane == 0) {
          s_best_v[wave] = v;
          s_best_i[wave] = ix;
        }
        __syncthreads();
        if (t == 0) {
          for (int q = 0; q < SK_WAVES; ++q)
            if (argmax_better(s_best_v[q], s_best_i[q], best_v, best_i)) {
              best_v = s_best_v[q];
              best_i = s_best_i[q];
            }
        }
        break;
      }
    }
    __syncthreads();
  }
#undef LLMK_SK_FEED
#undef LLMK_SK_FEED_NEXT
#undef LLMK_SK_X
#undef LLMK_SK_QKV
#undef LLMK_SK_ATT
#undef LLMK_SK_U

  // ---- greedy token: each workgroup's best, the last one to arrive reduces them ----
  if (threadIdx.x == 0) {
    st_dev(&p.head_val[w], best_v);
    st_dev(&p.head_idx[w], best_i);
    stores_done();
    s_last = (take_ticket(p.head_cnt) == (unsigned)(p.nwg - 1));
  }
  __syncthreads();
  if (!s_last) return;
  float v = -INFINITY;
  int ix = INT_MAX;
  for (int b = threadIdx.x; b < p.nwg; b += SK_THREADS) {
    const float bv = ld_dev(&p.head_val[b]);
    const int bi = ld_dev(&p.head_idx[b]);
    if (argmax_better(bv, bi, v, ix)) { v = bv; ix = bi; }
  }
  wave_argmax(v, ix);
  if (lane == 0) {
    s_best_v[wave] = v;
    s_best_i[wave] = ix;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = s_best_v[0];
    ix = s_best_i[0];
    for (int q = 1; q < SK_WAVES; ++q)
      if (argmax_better(s_best_v[q], s_best_i[q], v, ix)) { v = s_best_v[q]; ix = s_best_i[q]; }
    p.token_out[step] = ix;
    p.state->token = ix;
    p.state->pos = p.state->pos + 1;
    p.state->step = step + 1;
    reset_ticket(p.head_cnt);
  }
}

template <typename T, int HD>
static const void* step_fn() {
  return reinterpret_cast<const void*>(&step_kernel<T, HD>);
}

static const void* step_kernel_ptr(int kv_is_bf16, int hd) {
  switch (hd) {
#define LLMK_SK_CASE(H) \
  case H: return kv_is_bf16 ? step_fn<bf16_t, H>() : step_fn<float, H>();
    LLMK_SK_CASE(2) LLMK_SK_CASE(4) LLMK_SK_CASE(8) LLMK_SK_CASE(16) LLMK_SK_CASE(32) LLMK_SK_CASE(64)
    LLMK_SK_CASE(128) LLMK_SK_CASE(256)
#undef LLMK_SK_CASE
  }
  return nullptr;
}

int step_grid(int kv_is_bf16, int hd, int64_t vin_floats) {
  const void* fn = step_kernel_ptr(kv_is_bf16, hd);
  if (!fn) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, SK_THREADS, (size_t)vin_floats * sizeof(float)) !=
      hipSuccess)
    return 0;
  return per_cu >= 1 ? cus : 0;
}

hipError_t step_launch(const StepParams& p, int kv_is_bf16, int64_t vin_floats, hipStream_t s) {
  const void* fn = step_kernel_ptr(kv_is_bf16, p.hd);
  if (!fn || p.nwg < 1) return hipErrorInvalidValue;
  void* args[] = {const_cast<StepParams*>(&p)};
  return hipLaunchKernel(fn, dim3((unsigned)p.nwg), dim3(SK_THREADS), args, (size_t)vin_floats * sizeof(float), s);
}

}  // namespace llmk

namespace llmk {

// The layer table lives in the workspace; it is written by small kernels (layers passed by value, 8 at a
// time), so filling it needs no host-to-device copy and can sit in a captured graph.
__global__ void step_table_kernel(StepLayer* dst, const StepTableChunk chunk) {
  if (threadIdx.x < (unsigned)chunk.count) dst[chunk.first + threadIdx.x] = chunk.layers[threadIdx.x];
}

hipError_t step_table_launch(StepLayer* dst, const StepTableChunk& chunk, hipStream_t s) {
  hipLaunchKernelGGL(step_table_kernel, dim3(1), dim3(64), 0, s, dst, chunk);
  return hipGetLastError();
}

}  // namespace llmk
