// Split-context grouped-query decode attention for gfx950: the per-workgroup body, shared by the attention
// kernel and the persistent decode-step kernel.
//
// One query position; head h reads K/V head g = h / G (G = H / Hkv query heads share every K/V row, so
// each row is read from HBM once for all G of them). The context is cut into parts of consecutive
// tiles; a workgroup of 8 waves owns one (K/V head, part) and runs two tile streams of 4 waves, each
// taking every other tile of the part with an online softmax of its own.
//   - A tile of K and V rows is loaded cooperatively with 16-byte loads into registers while the
//     previous tile is being computed, then written to LDS (rows padded by 16 B so that a lane reading
//     its own row and lanes reading one row's consecutive elements are both bank-conflict free).
//   - Scores: wave w of a stream takes query heads w, w+4; lane t computes q . K[t] from LDS (q
//     broadcast from LDS), so no cross-lane reduction is needed per row. Softmax statistics are two
//     wave reductions.
//   - Output: lane groups take rows of the tile, lanes within a group own 16-byte slices of the head
//     dimension; the groups are summed once per part (xor shuffles) and the two streams are combined
//     through LDS.
//   - Each part writes (max, sum, unnormalised output) per head; the last workgroup of a K/V head merges
//     the parts by log-sum-exp in part order: m* = max m_c, out = sum_c e^(m_c - m*) o_c /
//     sum_c e^(m_c - m*) l_c.
// ("Inside the engine", "1. CausalLM": flash attention split across the context and reduced;
// "The forward pass end to end", "The code": the per-head softmax attention it computes.)
#pragma once

#include <float.h>

#include <type_traits>

#include "kernels.h"

namespace llmk {

constexpr int ATTN_THREADS = 512;
constexpr int ATTN_STREAMS = 2;                       // tile streams per workgroup
constexpr int ATTN_SWAVES = 4;                        // waves per stream
constexpr int ATTN_STHREADS = ATTN_SWAVES * 64;       // threads per stream
constexpr int ATTN_MAXG_PER_WAVE = 2;                 // query heads per wave (G <= 8)
static_assert(ATTN_THREADS % 128 == 0, "a thread's RoPE pair index is the same on every iteration for hd <= 256");

// positions per tile for a row of `row_bytes`: at most 64, tile of one of K/V at most 16 KiB
__host__ __device__ constexpr int attn_tile_rows(int row_bytes) {
  return (16384 / row_bytes) < 64 ? (16384 / row_bytes) : 64;
}

// The int8 cache (T = int8_t): rows of codes with one fp32 scale per (position, K/V head); its tiles are held
// in LDS as bf16 (every code is exact in bf16), so TS is the element type of the staged tiles.
template <typename T>
using attn_staged_t = typename std::conditional<std::is_same<T, int8_t>::value, bf16_t, T>::type;

// 16-byte vectors of the LDS tile buffer attn_block needs for cache element type T and head size HD
template <typename T, int HD>
__host__ __device__ constexpr int attn_tile_vecs() {
  using TS = attn_staged_t<T>;
  return ATTN_STREAMS * 2 * attn_tile_rows((HD * (int)sizeof(TS) + 15) / 16 * 16) *
         (((HD + 16 / (int)sizeof(TS) - 1) / (16 / (int)sizeof(TS))) + 1);
}

// Two int8 codes (bytes sh / 8 and sh / 8 + 1 of w) as a pair of bf16, the first in the low half: exact.
__device__ __forceinline__ uint32_t i8_pair_bf16(uint32_t w, int sh) {
  const float a = (float)(int8_t)(w >> sh), b = (float)(int8_t)(w >> (sh + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}


// (value, tag) pairs: the value's fp32 bits in the low word, the tag in the high word; one 8-byte store, so
// a reader sees both or neither
__device__ __forceinline__ void st_tag(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t v) { return (uint32_t)(v >> 32); }
__device__ __forceinline__ float val_of(uint64_t v) { return __uint_as_float((uint32_t)v); }

// Activations of the persistent step (x, q|k|v, the attention output, u) carry their tag in the two low
// mantissa bits of the fp32 value: 1 + the parity of the step within the call. Every such value is written
// once per step and the buffers are cleared (0) before a call, so a reader sees the current step's tag only
// on the current step's value. Dropping the two bits changes a value by less than 2^-21 of it; the hand-off
// moves 4 bytes a value instead of 8.
__device__ __forceinline__ uint32_t act_tag(uint32_t step) { return 1u + (step & 1u); }
__device__ __forceinline__ void st_act(uint32_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, (__float_as_uint(v) & ~3u) | tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_act(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool act_has(uint32_t b, uint32_t tag) { return (b & 3u) == tag; }
__device__ __forceinline__ float act_val(uint32_t b) { return __uint_as_float(b & ~3u); }

// Bounded wait: false once the wait has lasted longer than `ticks` of the 100 MHz real-time counter or
// another workgroup has given up (*err != 0); then *err is set, so every other waiter stops too.
constexpr uint64_t TAG_WAIT_TICKS = 20000000ull;   // 200 ms
__device__ __forceinline__ bool tag_wait_more(int32_t* err, uint64_t t0, unsigned& n) {
  __builtin_amdgcn_s_sleep(1);
  if ((++n & 15u) == 0u) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > TAG_WAIT_TICKS) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
  }
  return true;
}

// One workgroup's share of the attention: context part `part` of K/V head `kvh` of batch row `row` (row 0
// for a single sequence). Every thread of the workgroup (ATTN_THREADS) must call it with the same
// arguments; it returns at the same point for all of them. `tiles` is LDS of attn_tile_vecs<T, HD>()
// 16-byte vectors.
// TAG: the decode step's persistent form. q|k|v come as tagged activations from p.qkv_tag and are waited
// for until they carry p.tag; the merged output goes to p.out_tag tagged with p.tag.
template <typename T, int HD, bool TAG = false>
__device__ __forceinline__ void attn_block(const AttnParams& p, const int kvh, const int part, const int row,
                                           uint4* tiles) {
  constexpr bool Q8 = std::is_same<T, int8_t>::value;   // int8 codes, a scale per (position, K/V head)
  using TS = attn_staged_t<T>;                           // element type of the tiles in LDS
  constexpr int EPV = 16 / (int)sizeof(TS);              // staged elements per 16-byte vector
  constexpr int RV = (HD + EPV - 1) / EPV;               // vectors per row (a partial vector when HD < EPV)
  constexpr int ROWB = (HD * (int)sizeof(TS) + 15) / 16 * 16;
  constexpr int CH = attn_tile_rows(ROWB);               // positions per tile
  constexpr int RS = RV + 1;                             // padded row stride in vectors
  constexpr int EPG = 16 / (int)sizeof(T);               // cache elements per 16-byte load
  constexpr int RVG = (HD + EPG - 1) / EPG;              // loads per row
  static_assert(!Q8 || (HD % 16 == 0 && RV == 2 * RVG), "int8 rows are whole 16-code loads");
  constexpr int NVT = 2 * CH * RVG;                      // loads in a K+V tile
  constexpr int NVL = (NVT + ATTN_STHREADS - 1) / ATTN_STHREADS;   // per stream thread
  constexpr int LPV = RV;                                // V phase: lanes per row (one 16-B vector each)
  constexpr int RGV = 64 / LPV;                          // V phase: rows processed at once by a wave
  constexpr int HDP = HD < 4 ? 4 : HD;

  uint4 (&s_kv)[ATTN_STREAMS][2][CH][RS] = *reinterpret_cast<uint4 (*)[ATTN_STREAMS][2][CH][RS]>(tiles);
  // Scores on the matrix cores for bf16 K/V with HD a multiple of 32 and 64-position tiles: q is kept as
  // bf16 hi + lo parts (about 16 significant bits) and each score is taken twice (q hi . K + q lo . K) into fp32
  constexpr bool MF = sizeof(TS) == 2 && HD % 32 == 0 && CH == 16 * ATTN_SWAVES;
  __shared__ float s_q[MF ? 1 : 8][HDP];
  __shared__ __align__(16) bf16_t s_qh[MF ? 8 : 1][MF ? HD : 8];
  __shared__ __align__(16) bf16_t s_ql[MF ? 8 : 1][MF ? HD : 8];
  auto put_q = [&](int g, int e, float v) {
    if constexpr (MF) {
      bf16_t hi, lo;
      split_bf16(v, hi, lo);
      s_qh[g][e] = hi;
      s_ql[g][e] = lo;
    } else {
      s_q[g][e] = v;
    }
  };
  __shared__ float s_raw[TAG ? (8 + 2) * HDP : 1];     // TAG: this group's q heads, k and v as waited for
  __shared__ float s_p[ATTN_STREAMS][8][CH];
  __shared__ TS s_new[2][HDP];                           // the appended k and v row (decode), as staged
  __shared__ float s_newf[Q8 ? 2 : 1][Q8 ? HDP : 1];    // int8 cache: the new rows before quantization
  __shared__ float s_news[2];                            // and their scales
  __shared__ float s_sc[Q8 ? ATTN_STREAMS : 1][2][Q8 ? CH : 1];   // int8 cache: the tile rows' scales
  // stream 1's softmax state for the combine, in the tile buffer once the tiles are consumed (keeping it
  // out of the static LDS lets two workgroups share a CU)
  static_assert(16 + 8 * HDP <= 4 * attn_tile_vecs<T, HD>(), "combine state fits the tile buffer");
  float* const s_m1 = reinterpret_cast<float*>(tiles);
  float* const s_l1 = s_m1 + 8;
  float (&s_o1)[8][HDP] = *reinterpret_cast<float (*)[8][HDP]>(s_m1 + 16);
  __shared__ int s_last;

  const int G = p.H / p.Hkv;
  const bool batched = p.bstate != nullptr;
  const int ctx = batched ? p.bstate->pos[row] + 1 : (p.state ? p.state->pos + 1 : p.ctx);
  const int span = CH * p.sub_per_wg;
  const int tb = part * span;
  if (tb >= ctx) return;
  const int te = min(tb + span, ctx);

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int st = wv / ATTN_SWAVES;                       // tile stream of this wave
  const int wave = wv % ATTN_SWAVES;                     // wave within its stream
  const int stid = threadIdx.x % ATTN_STHREADS;          // thread within its stream
  const int64_t rstride = (int64_t)p.Hkv * HD;           // elements between positions
  // the row's slot region (contiguous pool), or its row of the block table (paged pool: tiles are a divisor of
  // the block, so every position of a tile sits in one block and the tile's rows are consecutive)
  const int32_t* const trow =
      p.pg.table ? p.pg.table + (batched ? (int64_t)p.bstate->slot[row] * p.pg.stride : 0) : nullptr;
  const int64_t rbase = batched && !trow ? (int64_t)p.bstate->slot[row] * p.slot_elems : 0;
  const T* Kb = static_cast<const T*>(p.k) + rbase + (int64_t)kvh * HD;
  const T* Vb = static_cast<const T*>(p.v) + rbase + (int64_t)kvh * HD;
  // int8 cache: scale of cache row r (of this slot's region, or of the store when paged) at [r * Hkv]
  const int64_t sbase = (rbase / rstride) * p.Hkv + kvh;
  const float* Ks = Q8 ? p.k_scale + sbase : nullptr;
  const float* Vs = Q8 ? p.v_scale + sbase : nullptr;
  const float* qkv_raw = p.qkv_raw ? p.qkv_raw + (batched ? (int64_t)row * p.qkv_stride : 0) : nullptr;
  unsigned* counters = p.counters + (batched ? (int64_t)row * p.Hkv : 0);
  const float scale = 1.0f / sqrtf((float)HD);

  // paged: the part's table entries (the first ATTN_TBL of them) are staged in LDS while the first tiles
  // load, so a later tile finds its block without a global load in front of its own loads
  constexpr int ATTN_TBL = 64;
  __shared__ int32_t s_tbl[ATTN_TBL];
  const int blk0 = trow ? (tb >> p.pg.shift) : 0;
  if (trow && (int)threadIdx.x < min(((te - 1) >> p.pg.shift) - blk0 + 1, ATTN_TBL))
    s_tbl[threadIdx.x] = trow[blk0 + threadIdx.x];
  // cache row of a tile's first position minus that position (0 for a contiguous slot)
  auto tile_base = [&](int T0, bool staged) -> int64_t {
    if (!trow) return 0;
    const int j = (T0 >> p.pg.shift) - blk0;
    const int32_t b = staged && j < ATTN_TBL ? s_tbl[j] : trow[T0 >> p.pg.shift];
    return (((int64_t)b << p.pg.shift) | (T0 & ((1 << p.pg.shift) - 1))) - T0;
  };

  // cooperative tile load by one stream: vector idx -> (K or V, row, vector); rows past te are clamped
  // to te - 1; a paged tile starts at the cache row of its first position
  uint4 reg[NVL];
  float sreg = 0.0f;                                     // int8 cache: one row's scale per thread < 2 CH
#define LLMK_LOAD_TILE(T0, STAGED)                                                                \
  const int64_t tile_row0 = tile_base((T0), (STAGED));                                             \
  _Pragma("unroll") for (int k = 0; k < NVL; ++k) {                                               \
    const int idx = stid + k * ATTN_STHREADS;                                                     \
    const int which = idx / (CH * RVG), rem = idx % (CH * RVG);                                   \
    const int t = min((T0) + rem / RVG, te - 1);                                                   \
    const T* src = (which == 0 ? Kb : Vb) + (tile_row0 + t) * rstride + (rem % RVG) * EPG;         \
    if (HD >= EPG) {                                                                              \
      reg[k] = idx < NVT ? gload_stream(src) : make_uint4(0, 0, 0, 0);                              \
    } else {                                                                                      \
      reg[k] = make_uint4(idx < NVT ? gload<uint32_t>(src) : 0u,                                  \
                          (idx < NVT && HD * (int)sizeof(T) >= 8) ? gload<uint32_t>(src + 4 / sizeof(T)) : 0u, \
                          0u, 0u);                                                                \
    }                                                                                             \
  }                                                                                               \
  if (Q8 && stid < 2 * CH) {                                                                      \
    const int t = min((T0) + stid % CH, te - 1);                                                   \
    sreg = (stid < CH ? Ks : Vs)[(tile_row0 + t) * p.Hkv];                                         \
  }
#define LLMK_STORE_TILE()                                                                         \
  _Pragma("unroll") for (int k = 0; k < NVL; ++k) {                                               \
    const int idx = stid + k * ATTN_STHREADS;                                                     \
    if (idx < NVT) {                                                                              \
      const int which = idx / (CH * RVG), rem = idx % (CH * RVG);                                 \
      if constexpr (Q8) {                                                                         \
        const uint4 c = reg[k];                                                                   \
        s_kv[st][which][rem / RVG][2 * (rem % RVG)] =                                             \
            make_uint4(i8_pair_bf16(c.x, 0), i8_pair_bf16(c.x, 16), i8_pair_bf16(c.y, 0), i8_pair_bf16(c.y, 16)); \
        s_kv[st][which][rem / RVG][2 * (rem % RVG) + 1] =                                         \
            make_uint4(i8_pair_bf16(c.z, 0), i8_pair_bf16(c.z, 16), i8_pair_bf16(c.w, 0), i8_pair_bf16(c.w, 16)); \
      } else {                                                                                    \
        s_kv[st][which][rem / RV][rem % RV] = reg[k];                                             \
      }                                                                                           \
    }                                                                                             \
  }                                                                                               \
  if (Q8 && stid < 2 * CH) s_sc[st][stid / CH][stid % CH] = sreg;

  const int n_tiles = (te - tb + CH - 1) / CH;
  // the first tile of each stream is requested before q is staged, so the two latencies overlap
  if (st < n_tiles) { LLMK_LOAD_TILE(tb + st * CH, false) }

  // q of the group into LDS. In the decode step q, k and v arrive unrotated (p.qkv_raw): every
  // workgroup rotates its q heads by the position, and the workgroup whose part holds that position
  // rotates k, rounds k and v to the cache dtype, appends them to the cache and patches its tile.
  const int pos = ctx - 1;
  const bool owner = (TAG || qkv_raw) && !p.no_append && pos >= tb && pos < te;
  // the RoPE row of this position: a thread's first (cos, sin) pair is requested before q is waited for
  constexpr int HALF = HD / 2;
  const float* tab = p.rope_table + (int64_t)pos * HALF * 2;
  const float2 cs_first = (TAG || qkv_raw) ? gload<float2>(tab + 2 * (threadIdx.x % HALF)) : make_float2(0.0f, 0.0f);
  if constexpr (TAG) {
    // this group's q heads, k and v: every thread loads its values, then reloads until each carries the
    // step's tag (the data is its own readiness signal)
    bool fl_failed = false;
    __syncthreads();
    const int nval = (G + 2) * HD;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    unsigned spins = 0;
    // a thread's values (at most QW of them, G <= 8 and HD <= 256) are loaded together and every one not yet
    // carrying the tag is reloaded in the same round
    constexpr int QW = (10 * HDP + ATTN_THREADS - 1) / ATTN_THREADS;
    uint32_t got[QW];
    int64_t gidx[QW];
#pragma unroll
    for (int k = 0; k < QW; ++k) {
      const int i = threadIdx.x + k * ATTN_THREADS;
      const int g = i / HD, e = i % HD;
      gidx[k] = g < G ? (int64_t)(kvh * G + g) * HD + e
                      : (int64_t)(p.H + (g - G) * p.Hkv) * HD + (int64_t)kvh * HD + e;
      got[k] = i < nval ? ld_act(p.qkv_tag + gidx[k]) : p.tag;
    }
    for (;;) {
      bool ready = true;
#pragma unroll
      for (int k = 0; k < QW; ++k) ready = ready && act_has(got[k], p.tag);
      if (ready || fl_failed) break;
      __builtin_amdgcn_s_sleep(8);   // about 0.2 us between reloads
      if (!tag_wait_more(p.err, t0, spins)) {
        fl_failed = true;
        break;
      }
#pragma unroll
      for (int k = 0; k < QW; ++k)
        if (!act_has(got[k], p.tag)) got[k] = ld_act(p.qkv_tag + gidx[k]);
    }
#pragma unroll
    for (int k = 0; k < QW; ++k) {
      const int i = threadIdx.x + k * ATTN_THREADS;
      if (i < nval) s_raw[i] = act_val(got[k]);
    }
    __syncthreads();
  }
  if (TAG || qkv_raw) {
    for (int i = threadIdx.x; i < (G + (owner ? 1 : 0)) * HALF; i += ATTN_THREADS) {
      const int g = i / HALF, j = i % HALF;
      const int ia = p.rope_layout == 0 ? j : 2 * j;
      const int ib = p.rope_layout == 0 ? j + HALF : 2 * j + 1;
      // ATTN_THREADS is a multiple of HALF, so j is this thread's prefetched pair on every iteration
      const float cs = cs_first.x, sn = cs_first.y;
      float a, b;
      if constexpr (TAG) {
        a = s_raw[g * HD + ia];
        b = s_raw[g * HD + ib];
      } else {
        const float* src = g < G ? qkv_raw + (int64_t)(kvh * G + g) * HD
                                 : qkv_raw + (int64_t)p.H * HD + (int64_t)kvh * HD;   // this head's k
        a = ld_dev(src + ia);
        b = ld_dev(src + ib);
      }
      const float ra = a * cs - b * sn, rb = a * sn + b * cs;
      if (g < G) {
        put_q(g, ia, ra);
        put_q(g, ib, rb);
      } else if constexpr (Q8) {
        s_newf[0][ia] = ra;
        s_newf[0][ib] = rb;
      } else {
        store_elem<T>(&s_new[0][0], ia, ra);
        store_elem<T>(&s_new[0][0], ib, rb);
      }
    }
    if (owner) {
      for (int e = threadIdx.x; e < HD; e += ATTN_THREADS) {
        float val;
        if constexpr (TAG) val = s_raw[(G + 1) * HD + e];
        else val = ld_dev(qkv_raw + (int64_t)(p.H + p.Hkv) * HD + (int64_t)kvh * HD + e);
        if constexpr (Q8) s_newf[1][e] = val;
        else store_elem<T>(&s_new[1][0], e, val);
      }
    }
    __syncthreads();
    if (owner) {
      const int64_t crow = trow ? kv_block_row(trow, p.pg.shift, pos) : (int64_t)pos;   // cache row of pos
      const int64_t off = crow * p.Hkv * HD + (int64_t)kvh * HD;
      if constexpr (Q8) {
        // wave w < 2 quantizes the new k (w = 0) or v row: s = max|x| / 127, codes rint(x / s) clamped to 127
        if (wv < 2) {
          float amax = 0.0f;
          for (int e = lane; e < HD; e += 64) amax = fmaxf(amax, fabsf(s_newf[wv][e]));
          const float sc = wave_max_dpp(amax) / 127.0f;
          int8_t* dst = static_cast<int8_t*>(wv == 0 ? p.k_w : p.v_w) + rbase + off;
          for (int e = lane; e < HD; e += 64) {
            const float r = sc > 0.0f ? fminf(fmaxf(rintf(s_newf[wv][e] / sc), -127.0f), 127.0f) : 0.0f;
            dst[e] = (int8_t)r;
            s_new[wv][e] = (bf16_t)(__float_as_uint(r) >> 16);
          }
          if (lane == 0) {
            s_news[wv] = sc;
            (wv == 0 ? p.k_scale_w : p.v_scale_w)[(rbase / rstride + crow) * p.Hkv + kvh] = sc;
          }
        }
        __syncthreads();
      } else {
        for (int e = threadIdx.x; e < 2 * HD; e += ATTN_THREADS) {
          const int w = e / HD, ee = e % HD;
          (w == 0 ? static_cast<T*>(p.k_w) : static_cast<T*>(p.v_w))[rbase + off + ee] = s_new[w][ee];
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < G * HD; i += ATTN_THREADS) put_q(i / HD, i % HD, p.q[(int64_t)kvh * G * HD + i]);
  }

  // per wave and query head: running max and sum (uniform), and a partial output per lane for the
  // EPV elements of vector `vl` over the rows of row group `rg` (reduced over row groups at the end)
  const int vl = lane % LPV, rg = lane / LPV;
  float m_run[ATTN_MAXG_PER_WAVE], l_run[ATTN_MAXG_PER_WAVE], o[ATTN_MAXG_PER_WAVE][EPV];
#pragma unroll
  for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi) {
    m_run[gi] = -INFINITY;
    l_run[gi] = 0.0f;
#pragma unroll
    for (int k = 0; k < EPV; ++k) o[gi][k] = 0.0f;
  }

  // stream st takes tiles st, st + 2, st + 4, ... of the part; every thread runs all iterations so
  // that the barriers match, a stream past its last tile idles
  const int iters = (n_tiles + ATTN_STREAMS - 1) / ATTN_STREAMS;
  for (int it = 0; it < iters; ++it) {
    const int t0 = tb + (it * ATTN_STREAMS + st) * CH;
    const bool act = t0 < te;
    __syncthreads();                       // previous tiles fully consumed (and q in LDS on entry)
    if (act) { LLMK_STORE_TILE() }
    __syncthreads();
    if (owner) {                           // the appended position: use the new row, not the stale one
      if (act && pos >= t0 && pos < t0 + CH) {
        for (int e = stid; e < 2 * HD; e += ATTN_STHREADS) {
          const int w = e / HD, ee = e % HD;
          reinterpret_cast<TS*>(&s_kv[st][w][pos - t0][0])[ee] = s_new[w][ee];
        }
        if (Q8 && stid < 2) s_sc[st][stid][pos - t0] = s_news[stid];
      }
      __syncthreads();
    }
    {
      const int tn = t0 + ATTN_STREAMS * CH;
      if (tn < te) { LLMK_LOAD_TILE(tn, true) }   // next tile in flight while this one is computed
    }
    const int n = act ? min(CH, te - t0) : 0;

    // scores and softmax statistics: wave w takes heads w, w + 4; lane t scores position t0 + t
    if constexpr (MF) {
      // S = Q K^T, 16 x 16 blocks: wave w of the stream takes positions 16w .. 16w + 15 of the tile for
      // every head (lane l: q row l % 16 and K row 16w + l % 16, dims 8 (l / 16) .. + 7 of each 32-wide step;
      // result: heads 4 (l / 16) .. + 3 of position 16w + l % 16); the scores go to s_p
      static_assert(CH == 16 * ATTN_SWAVES, "one 16-position block per wave");
      if (act) {
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const int m = lane & 15, kg = lane >> 4;
        const int prow = wave * 16 + m;
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks) {
          const uint4 kb = s_kv[st][0][prow][ks * 4 + kg];
          const uint4 qh = m < G ? *reinterpret_cast<const uint4*>(&s_qh[m][ks * 32 + 8 * kg]) : make_uint4(0, 0, 0, 0);
          const uint4 ql = m < G ? *reinterpret_cast<const uint4*>(&s_ql[m][ks * 32 + 8 * kg]) : make_uint4(0, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qh), __builtin_bit_cast(bf16x8_t, kb),
                                                         acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ql), __builtin_bit_cast(bf16x8_t, kb),
                                                         acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int g = 4 * kg + i;
          if (g < G) s_p[st][g][prow] = prow < n ? acc[i] * (Q8 ? scale * s_sc[st][0][prow] : scale) : -INFINITY;
        }
      }
      __syncthreads();
    }
    float alpha_g[ATTN_MAXG_PER_WAVE];
#pragma unroll
    for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi) {
      const int g = wave + gi * ATTN_SWAVES;
      alpha_g[gi] = 1.0f;
      if (g < G && act) {
        float s = -INFINITY;
        if constexpr (MF) {
          s = s_p[st][g][lane];
        } else if (lane < CH) {
          float part8[EPV];
#pragma unroll
          for (int e = 0; e < EPV; ++e) part8[e] = 0.0f;
          const float* qg = s_q[g];
#pragma unroll
          for (int v = 0; v < RV; ++v) {
            float kf[EPV];
            if constexpr (sizeof(TS) == 2) unpack<bf16_t, 8>(s_kv[st][0][lane][v], kf);
            else unpack<float, 4>(s_kv[st][0][lane][v], kf);
#pragma unroll
            for (int e = 0; e < EPV; ++e)
              if (v * EPV + e < HD) part8[e] = fmaf(qg[v * EPV + e], kf[e], part8[e]);
          }
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < EPV; ++e) dot += part8[e];
          if (lane < n) s = dot * (Q8 ? scale * s_sc[st][0][lane] : scale);
        }
        const float m_new = fmaxf(m_run[gi], wave_max_dpp(s));
        const float pr = (lane < n) ? expf(s - m_new) : 0.0f;
        const float alpha = expf(m_run[gi] - m_new);
        l_run[gi] = l_run[gi] * alpha + wave_sum_dpp(pr);
        m_run[gi] = m_new;
        alpha_g[gi] = alpha;
        if (lane < CH) s_p[st][g][lane] = pr;
      }
    }
    __syncthreads();
    // o = alpha o + sum_t p_t V[t]: lane (rg, vl) accumulates rows rg, rg + RGV, ... of the tile
#pragma unroll
    for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi) {
      const int g = wave + gi * ATTN_SWAVES;
      if (g < G && act) {
#pragma unroll
        for (int k = 0; k < EPV; ++k) o[gi][k] *= alpha_g[gi];
#pragma unroll 4
        for (int t = rg; t < n; t += RGV) {
          const float pt = Q8 ? s_p[st][g][t] * s_sc[st][1][t] : s_p[st][g][t];
          float vf[EPV];
          if constexpr (sizeof(TS) == 2) unpack<bf16_t, 8>(s_kv[st][1][t][vl], vf);
          else unpack<float, 4>(s_kv[st][1][t][vl], vf);
#pragma unroll
          for (int k = 0; k < EPV; ++k) o[gi][k] = fmaf(pt, vf[k], o[gi][k]);
        }
      }
    }
  }
#undef LLMK_LOAD_TILE
#undef LLMK_STORE_TILE

  // reduce the partial outputs over the row groups of each wave (xor shuffles, fixed order)
#pragma unroll
  for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi)
#pragma unroll
    for (int k = 0; k < EPV; ++k)
#pragma unroll
      for (int off = LPV; off < 64; off <<= 1) o[gi][k] += __shfl_xor(o[gi][k], off, 64);

  // ---- stream 1 hands its (max, sum, output) to stream 0 through LDS (the tile buffer: every wave is done
  // with the tiles first) ----
  __syncthreads();
  if (st == 1) {
#pragma unroll
    for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi) {
      const int g = wave + gi * ATTN_SWAVES;
      if (g < G) {
        if (lane == 0) {
          s_m1[g] = m_run[gi];
          s_l1[g] = l_run[gi];
        }
        if (rg == 0) {
#pragma unroll
          for (int k = 0; k < EPV; ++k)
            if (vl * EPV + k < HD) s_o1[g][vl * EPV + k] = o[gi][k];
        }
      }
    }
  }
  __syncthreads();

  // ---- this part's (max, sum, output) per head: stream 0 combines the two streams in LDS (each element
  // read and rewritten by the same lane), then every thread writes consecutive floats of the part ----
  if (st == 0) {
#pragma unroll
    for (int gi = 0; gi < ATTN_MAXG_PER_WAVE; ++gi) {
      const int g = wave + gi * ATTN_SWAVES;
      if (g < G) {
        const float m1 = s_m1[g];                        // -inf when stream 1 had no tile
        const float l1 = s_l1[g];
        const float ms = fmaxf(m_run[gi], m1);
        const float w0 = expf(m_run[gi] - ms);
        const float w1 = m1 == -INFINITY ? 0.0f : expf(m1 - ms);
        if (rg == 0) {
#pragma unroll
          for (int k = 0; k < EPV; ++k) {
            const int e = vl * EPV + k;
            if (e < HD) s_o1[g][e] = fmaf(s_o1[g][e], w1, o[gi][k] * w0);
          }
        }
        if (lane == 0) {
          s_m1[g] = ms;
          s_l1[g] = fmaf(l1, w1, l_run[gi] * w0);
        }
      }
    }
  }
  __syncthreads();
  const int64_t pstride = HD + 2;
  if constexpr (TAG) {
    // this part's (max, sum, output) per head as (value, part tag) pairs; a merging workgroup waits for them
    uint64_t* PT = p.part_tagged + ((int64_t)kvh * p.n_parts + part) * G * pstride;
    for (int i = threadIdx.x; i < G * pstride; i += ATTN_THREADS) {
      const int g = i / pstride, j = i % pstride;
      st_tag(&PT[i], j == 0 ? s_m1[g] : j == 1 ? s_l1[g] : s_o1[g][j - 2], p.part_tag);
    }
    __syncthreads();
    return;
  }
  float* part_base = p.part + (batched ? (int64_t)row * p.Hkv * p.n_parts * G * pstride : 0);
  float* P = part_base + ((int64_t)kvh * p.n_parts + part) * G * pstride;
  for (int i = threadIdx.x; i < G * pstride; i += ATTN_THREADS) {
    const int g = i / pstride, j = i % pstride;
    st_dev(&P[i], j == 0 ? s_m1[g] : j == 1 ? s_l1[g] : s_o1[g][j - 2]);
  }

  // ---- last workgroup of this K/V head: log-sum-exp merge of the parts, in part order ----
  stores_done();
  __syncthreads();
  const int np = (ctx + span - 1) / span;
  if (threadIdx.x == 0) {
    s_last = (take_ticket(&counters[kvh]) == (unsigned)(np - 1));
    // the last workgroup re-arms the counter before any of its output can be seen, so a reader of the
    // output never finds the counter still counting
    if (s_last) {
      reset_ticket(&counters[kvh]);
      stores_done();
    }
  }
  __syncthreads();
  if (!s_last) return;
  // every thread issues all its loads at once (max, sum and its output element of every part), so the
  // merge costs one round trip; parts are combined in part order
  const float* PB = part_base + (int64_t)kvh * p.n_parts * G * pstride;
  const int64_t cstride = (int64_t)G * pstride;
  for (int idx = threadIdx.x; idx < G * HD; idx += ATTN_THREADS) {
    const int g = idx / HD, e = idx % HD;
    const float* pg = PB + (int64_t)g * pstride;
    float mc[ATTN_MAX_PARTS], lc[ATTN_MAX_PARTS], oc[ATTN_MAX_PARTS];
#pragma unroll
    for (int c = 0; c < ATTN_MAX_PARTS; ++c) {
      const int cc = c < np ? c : np - 1;
      mc[c] = ld_dev(pg + cc * cstride + 0);
      lc[c] = ld_dev(pg + cc * cstride + 1);
      oc[c] = ld_dev(pg + cc * cstride + 2 + e);
    }
    float ms = -INFINITY;
#pragma unroll
    for (int c = 0; c < ATTN_MAX_PARTS; ++c) ms = c < np ? fmaxf(ms, mc[c]) : ms;
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int c = 0; c < ATTN_MAX_PARTS; ++c) {
      if (c < np) {
        const float w = expf(mc[c] - ms);
        L = fmaf(lc[c], w, L);
        O = fmaf(oc[c], w, O);
      }
    }
    const int64_t oi = (int64_t)(kvh * G + g) * HD + e;
    if constexpr (TAG) {
      st_act(p.out_tag + oi, O / L, p.tag);
    } else if (p.out_hi) {
      bf16_t hi, lo;
      split_bf16(O / L, hi, lo);
      p.out_hi[(int64_t)row * p.H * HD + oi] = hi;
      p.out_lo[(int64_t)row * p.H * HD + oi] = lo;
    } else {
      st_dev(&p.out[oi], O / L);
    }
  }
}

// TAG form of the merge: query head g of K/V head kvh, by a workgroup of its own. It waits for the
// (max, sum, output) of all n_parts parts to carry p.part_tag, combines them by log-sum-exp and writes the
// head's output as activations tagged p.tag. Thread t takes output element t % HD over the parts
// c = t / HD, t / HD + NS, ... (NS = ATTN_THREADS / HD subsets); the subsets are combined in order through
// LDS. Every thread of the workgroup must call it.
template <int HD>
__device__ __forceinline__ void attn_merge_tagged(const AttnParams& p, const int kvh, const int g, const int n_parts) {
  constexpr int NS = ATTN_THREADS / HD;                         // part subsets
  constexpr int NPP = (ATTN_MAX_PARTS + NS - 1) / NS;           // parts per thread, at most
  __shared__ float s_pm[ATTN_MAX_PARTS], s_pl[ATTN_MAX_PARTS];  // each part's max and sum
  __shared__ float s_m[ATTN_THREADS], s_l[ATTN_THREADS], s_o[ATTN_THREADS];
  const int G = p.H / p.Hkv;
  const int64_t pstride = HD + 2;
  const int e = threadIdx.x % HD, sub = threadIdx.x / HD;
  const uint64_t* PB = p.part_tagged + ((int64_t)kvh * n_parts * G + g) * pstride;
  const int64_t cstride = (int64_t)G * pstride;
  bool failed = false;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  unsigned spins = 0;
  // a part's (max, sum): thread c < 2 n_parts waits for one of them
  if (threadIdx.x < 2 * n_parts) {
    const int c = threadIdx.x >> 1;
    const uint64_t* src = PB + c * cstride + (threadIdx.x & 1);
    uint64_t v = ld_tag(src);
    while (tag_of(v) != p.part_tag && !failed) {
      if (!tag_wait_more(p.err, t0, spins)) failed = true;
      v = ld_tag(src);
    }
    ((threadIdx.x & 1) ? s_pl : s_pm)[c] = val_of(v);
  }
  // this thread's output element over its parts: every part not yet carrying the tag is reloaded in the
  // same round, so the wait ends one round trip after the last part lands
  uint64_t o[NPP];
#pragma unroll
  for (int k = 0; k < NPP; ++k) {
    const int c = sub + k * NS;
    o[k] = c < n_parts ? ld_tag(PB + c * cstride + 2 + e) : ((uint64_t)p.part_tag << 32);
  }
  for (;;) {
    bool ready = true;
#pragma unroll
    for (int k = 0; k < NPP; ++k) ready = ready && tag_of(o[k]) == p.part_tag;
    if (ready || failed) break;
    if (!tag_wait_more(p.err, t0, spins)) {
      failed = true;
      break;
    }
#pragma unroll
    for (int k = 0; k < NPP; ++k) {
      const int c = sub + k * NS;
      if (tag_of(o[k]) != p.part_tag) o[k] = ld_tag(PB + c * cstride + 2 + e);
    }
  }
  __syncthreads();
  float ms = -INFINITY;
#pragma unroll
  for (int k = 0; k < NPP; ++k)
    if (sub + k * NS < n_parts) ms = fmaxf(ms, s_pm[sub + k * NS]);
  float L = 0.0f, O = 0.0f;
#pragma unroll
  for (int k = 0; k < NPP; ++k) {
    const int c = sub + k * NS;
    if (c < n_parts) {
      const float w = expf(s_pm[c] - ms);
      L = fmaf(s_pl[c], w, L);
      O = fmaf(val_of(o[k]), w, O);
    }
  }
  s_m[threadIdx.x] = ms;
  s_l[threadIdx.x] = L;
  s_o[threadIdx.x] = O;
  __syncthreads();
  if (threadIdx.x < HD) {
    float M = -INFINITY;
    for (int q = 0; q < NS && q < n_parts; ++q) M = fmaxf(M, s_m[q * HD + e]);
    float LL = 0.0f, OO = 0.0f;
    for (int q = 0; q < NS && q < n_parts; ++q) {
      const float w = expf(s_m[q * HD + e] - M);
      LL = fmaf(s_l[q * HD + e], w, LL);
      OO = fmaf(s_o[q * HD + e], w, OO);
    }
    st_act(p.out_tag + (int64_t)(kvh * G + g) * HD + e, OO / LL, p.tag);
  }
  __syncthreads();
}

}  // namespace llmk
