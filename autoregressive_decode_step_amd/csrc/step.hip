// The whole decode step of one sequence as one persistent kernel (gfx950).
//
// A step is a chain of operations, each needing all of the previous one's output: RMSNorm + q|k|v,
// attention, o + residual, RMSNorm + gate|up, down + residual, per layer, then the final norm, the head
// and the greedy token ("The forward pass end to end", "What a forward step does"). Launched one kernel
// per operation, every operation pays a launch, a ramp-up and a drain, about as long as a small projection
// itself. Here one workgroup per CU runs the whole step.
//
// Weight stream. Every projection y = W v is cut into row ranges, one per workgroup; inside a workgroup
// wave w takes rows w, w + 8, ... (gate|up: the gate row and the up row of outputs w, w + 8, ...). A wave
// reads a row as 16-byte loads per lane (512 bf16 per load, coalesced) and dots it with the staged input
// vector in LDS. Each wave keeps SK_R loads in flight in a register ring, and the ring runs on from one
// operation into the next: while a workgroup waits for the next operation's input, the first SK_R loads of
// that operation's weights are already on their way, so HBM stays busy across the step's dependencies
// ("Inside the engine", "4. The pipelined decode": keep the device busy between the step's pieces).
// Every operation's load count per wave is padded to a multiple of SK_R (the padding re-reads the wave's
// last row, from cache, and is not used), so ring slot indices are compile-time constants.
//
// Hand-off without barriers. Every activation one workgroup writes and another reads (q|k|v, the
// attention output, x after each residual add, u) is stored as an fp32 word whose two low mantissa bits
// hold a tag, 1 + the parity of the step within the call (the attention's partial results, whose count
// changes with the context, as 8-byte (value, tag) pairs with a tag per step and layer). A reader loads
// what it needs with device-scope loads (past the non-coherent L2 of its XCD) and reloads until every value
// carries the current tag: the data itself is the signal, so a dependency costs one round trip and no
// writer ever waits for its stores. The buffers are cleared before each call. Every wait is bounded (200 ms of the real-time counter); a
// workgroup that gives up sets an error flag that stops every other waiter, and the host reports a device
// error.
//
// Norms. RMSNorm(x) * g is applied as (x * g) staged in LDS and the scalar rsqrt(mean(x^2) + eps) applied
// to each row's dot product, so the dots start as soon as x is staged.
//
// int8 weight packs (QW). The same stream over the codes of the library's int8 packs: a lane's 16-byte load
// holds 16 codes of one group, so a wave load covers 1,024 inputs, and a second ring of 4-byte loads brings
// each slot's group scale; a slot's 16 products are summed, then scaled ("Inside the engine", "1. CausalLM":
// decode reads packed weights).
#include <limits.h>

#include <type_traits>

#include "attn_block.h"

namespace llmk {

constexpr int SK_THREADS = ATTN_THREADS;   // 512: 8 waves
constexpr int SK_WAVES = SK_THREADS / 64;
static_assert(SK_WAVES == 8 && STEP_MAX_WAVE_ROWS == 2 * 64, "a wave keeps its row results in two registers of 64 lanes");
constexpr int SK_R = 8;                     // weight loads in flight per lane
constexpr int SK_SEG = 512;                 // elements of one wave load (64 lanes x 8 bf16)
// int8 weight packs (QW): a lane loads 16 codes, so a wave load covers 1,024 elements of a row, and every
// 16 codes of a lane lie in one group of SK_QG inputs with its own fp32 scale
constexpr int SK_SEG_Q = 1024;
constexpr int SK_QG = 128;
template <bool QW>
__host__ __device__ constexpr int sk_seg() {
  return QW ? SK_SEG_Q : SK_SEG;
}
constexpr int SK_PASS = 4;                  // float4 groups per thread staged per round trip

enum { OP_QKV = 0, OP_O = 1, OP_GU = 2, OP_DN = 3, OP_HEAD = 4 };

struct SkRange {
  int lo, n;
};

__device__ __forceinline__ SkRange sk_range(int rows, int w, int nwg) {
  const int lo = (int)(((int64_t)rows * w) / nwg);
  const int hi = (int)(((int64_t)rows * (w + 1)) / nwg);
  return {lo, hi - lo};
}

// this workgroup's rows of every projection
struct SkRows {
  SkRange q, k, v;   // rows of wq, wk, wv
  SkRange d;         // outputs of o and down (and the residual rows it keeps)
  SkRange f;         // outputs of gate|up
  SkRange h;         // rows of the head
};

// the layer table, staged in LDS once
struct SkLayer {
  const bf16_t* w[7];
  const float* g1;
  const float* g2;
  void* k;
  void* v;
};

// One projection as one wave streams it. A row is 2^sh load slots (its loads rounded up to a power of
// two; the extra slots re-read the row's last 16 bytes, which meet zeros of the staged input); load slot u
// of the wave is slot u & (2^sh - 1) of wave-local row u >> sh.
struct SkScales {      // int8 packs: the scales of the first rows below (K / SK_QG per row)
  const float* s0;
  const float* s1;
  const float* s2;
};
struct SkNoScales {};
template <bool QW>
struct SkOp : std::conditional<QW, SkScales, SkNoScales>::type {
  int kind, l;
  int K, sh;          // row length, log2 of the load slots per row
  int nrows, npos;    // rows of this wave, its load slots (nrows << sh rounded up to SK_R; 0: none)
  int n0, n01;        // QKV: the workgroup's rows of wq, of wq and wk (else larger than any row)
  int kmax;           // byte offset of a row's last 16-byte slice
  const char* m0;     // the workgroup's first row of wq / gate / the matrix (bf16 elements, or int8 codes)
  const char* m1;     // of wk / up
  const char* m2;     // of wv
};

// c ? a : b on values (a conditional on two struct members would select between their addresses and keep
// the struct in memory)
template <typename V>
__device__ __forceinline__ V sk_sel(bool c, V a, V b) {
  return c ? a : b;
}

// a pointer every lane holds the same value of, moved to scalar registers
template <typename P>
__device__ __forceinline__ P* sk_uniform(P* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// The workgroup's first row `lo` of a [rows][K] matrix: bf16 elements, or the codes of an int8 pack (whose
// scales, K / SK_QG per row, follow all rows * K codes; *sc gets the first row's).
template <bool QW>
__device__ __forceinline__ const char* sk_rows_of(const bf16_t* m, int rows, int K, int lo, const float** sc) {
  if constexpr (QW) {
    const char* b = reinterpret_cast<const char*>(sk_uniform(m));
    *sc = reinterpret_cast<const float*>(b + (int64_t)rows * K) + (int64_t)lo * (K / SK_QG);
    return b + (int64_t)lo * K;
  } else {
    return reinterpret_cast<const char*>(sk_uniform(m) + (int64_t)lo * K);
  }
}

template <bool QW>
__device__ __forceinline__ SkOp<QW> sk_op(const StepParams& p, const SkRows& R, const SkLayer* lt, int o, int wave) {
  SkOp<QW> f;
  int rw;
  f.n0 = f.n01 = INT_MAX;
  const float* sdummy;
  const float** s0 = &sdummy;
  const float** s1 = &sdummy;
  const float** s2 = &sdummy;
  if constexpr (QW) {
    s0 = &f.s0;
    s1 = &f.s1;
    s2 = &f.s2;
  }
  if (o >= 4 * p.n_layer) {
    f.kind = OP_HEAD;
    f.l = 0;
    f.K = p.d;
    f.m0 = sk_rows_of<QW>(p.w_out, p.V, p.d, R.h.lo, s0);
    rw = R.h.n;
  } else {
    f.l = o >> 2;
    f.kind = o & 3;
    const SkLayer& Ly = lt[f.l];
    switch (f.kind) {
      case OP_QKV:
        f.K = p.d;
        f.m0 = sk_rows_of<QW>(Ly.w[0], p.qd, p.d, R.q.lo, s0);
        f.m1 = sk_rows_of<QW>(Ly.w[1], p.kvd, p.d, R.k.lo, s1);
        f.m2 = sk_rows_of<QW>(Ly.w[2], p.kvd, p.d, R.v.lo, s2);
        f.n0 = R.q.n;
        f.n01 = R.q.n + R.k.n;
        rw = R.q.n + R.k.n + R.v.n;
        break;
      case OP_O:
        f.K = p.qd;
        f.m0 = sk_rows_of<QW>(Ly.w[3], p.d, p.qd, R.d.lo, s0);
        rw = R.d.n;
        break;
      case OP_GU:
        f.K = p.d;
        f.m0 = sk_rows_of<QW>(Ly.w[4], p.F, p.d, R.f.lo, s0);
        f.m1 = sk_rows_of<QW>(Ly.w[5], p.F, p.d, R.f.lo, s1);
        rw = R.f.n;
        break;
      default:
        f.K = p.F;
        f.m0 = sk_rows_of<QW>(Ly.w[6], p.d, p.F, R.d.lo, s0);
        rw = R.d.n;
        break;
    }
  }
  if (f.kind != OP_QKV) {
    const bool gu = f.kind == OP_GU;
    f.m1 = f.m2 = sk_sel<const char*>(gu, f.m1, f.m0);
    if constexpr (QW) f.s1 = f.s2 = sk_sel<const float*>(gu, f.s1, f.s0);
  }
  const int lpr = (f.K + sk_seg<QW>() - 1) / sk_seg<QW>();
  f.sh = 0;
  while ((1 << f.sh) < lpr) ++f.sh;
  f.kmax = QW ? f.K - 16 : 2 * (f.K - 8);
  const int mine = rw > wave ? (rw - wave + SK_WAVES - 1) / SK_WAVES : 0;
  f.nrows = f.kind == OP_GU ? 2 * mine : mine;
  f.npos = ((f.nrows << f.sh) + SK_R - 1) / SK_R * SK_R;
  return f;
}

// address of load slot u of op f for this lane (slots past the wave's rows re-read its last row); with int8
// packs *sa gets the address of the slot's scale (the group of the lane's 16 codes)
template <bool QW>
__device__ __forceinline__ const char* sk_addr(const SkOp<QW>& f, int u, int wave, int lane16, const float** sa) {
  const int r = min(u >> f.sh, f.nrows - 1);
  const int c = u & ((1 << f.sh) - 1);
  const int q = wave + SK_WAVES * r;
  const int j = wave + SK_WAVES * (r >> 1);
  const bool gu = f.kind == OP_GU;
  const char* m0 = f.m0;
  const char* m1 = f.m1;
  const char* m2 = f.m2;
  const int n0 = f.n0, n01 = f.n01;
  const char* base = sk_sel(gu, sk_sel((r & 1) != 0, m1, m0), sk_sel(q < n0, m0, sk_sel(q < n01, m1, m2)));
  const int row = sk_sel(gu, j, sk_sel(q < n0, q, sk_sel(q < n01, q - n0, q - n01)));
  if constexpr (QW) {
    const int off = min(c * SK_SEG_Q + lane16, f.kmax);
    const float* sb = sk_sel(gu, sk_sel((r & 1) != 0, f.s1, f.s0), sk_sel(q < n0, f.s0, sk_sel(q < n01, f.s1, f.s2)));
    *sa = sb + (int64_t)row * (f.K / SK_QG) + off / SK_QG;
    return base + (int64_t)row * f.K + off;
  } else {
    const int off = min(c * (SK_SEG * 2) + lane16, f.kmax);
    return reinterpret_cast<const char*>(reinterpret_cast<const bf16_t*>(base) + (int64_t)row * f.K) + off;
  }
}

// LDS position of input element e (e % 4 == 0 for a float4 group). bf16 rows: lane l's 8 elements of
// segment c sit as two float4 at c*512 + l*4 and c*512 + 256 + l*4; int8 rows: lane l's 16 elements of
// segment c as four float4 at c*1024 + k*256 + l*4. Every read of a segment is contiguous over the lanes.
template <bool QW>
__device__ __forceinline__ int sk_vin_pos(int e) {
  if constexpr (QW) {
    const int c = e >> 10, r = e & 1023;
    return (c << 10) | (((r >> 2) & 3) << 8) | ((r >> 4) << 2) | (r & 3);
  } else {
    const int c = e >> 9, r = e & 511;
    return (c << 9) | (((r >> 2) & 1) << 8) | ((r >> 3) << 2) | (r & 3);
  }
}

// Stage an input vector of n fp32 values into LDS (permuted; zeros up to the padded row length npad):
// src_tag = tagged activations waited for, or src_emb = a bf16 row (no wait). gain: multiply by it.
// res: copy elements [res_lo, res_lo + res_n) unmultiplied to res. Returns this thread's sum of squares.
template <bool QW>
__device__ __forceinline__ float sk_stage(const uint32_t* src_tag, const bf16_t* src_emb, int n, int npad,
                                          uint32_t tag, const float* gain, float* res, int res_lo, int res_n,
                                          float* vin, int32_t* err, bool& failed) {
  const int t = threadIdx.x;
  const int ng = (n / 4 + SK_THREADS - 1) / SK_THREADS;   // float4 groups per thread (uniform)
  float ss = 0.0f;
  for (int k0 = 0; k0 < ng; k0 += SK_PASS) {
    float v[SK_PASS][4];
    float4 g[SK_PASS];
    if (gain) {
#pragma unroll
      for (int k = 0; k < SK_PASS; ++k) {
        const int e = 4 * (t + (k0 + k) * SK_THREADS);
        if (k0 + k < ng && e < n) g[k] = gload<float4>(gain + e);
      }
    }
    if (src_emb) {
#pragma unroll
      for (int k = 0; k < SK_PASS; ++k) {
        const int e = 4 * (t + (k0 + k) * SK_THREADS);
        if (k0 + k < ng && e < n) {
          const uint2 w = gload<uint2>(src_emb + e);
          v[k][0] = bf16_lo(w.x);
          v[k][1] = bf16_hi(w.x);
          v[k][2] = bf16_lo(w.y);
          v[k][3] = bf16_hi(w.y);
        }
      }
    } else {
      // device-scope 16-byte loads (sc1), four tagged values each; past n the loads return zeros
      __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(src_tag), (short)0, n * 4, 0x00020000);
      uint4 a[SK_PASS];
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      unsigned spins = 0;
      for (;;) {
#pragma unroll
        for (int k = 0; k < SK_PASS; ++k) {
          if (k0 + k < ng) {
            const int off = 16 * (t + (k0 + k) * SK_THREADS);
            a[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16));
          }
        }
        bool ready = true;
#pragma unroll
        for (int k = 0; k < SK_PASS; ++k) {
          const int e = 4 * (t + (k0 + k) * SK_THREADS);
          if (k0 + k < ng && e < n)
            ready = ready && act_has(a[k].x, tag) && act_has(a[k].y, tag) && act_has(a[k].z, tag) && act_has(a[k].w, tag);
        }
        if (ready || failed) break;
        __builtin_amdgcn_s_sleep(8);   // about 0.2 us between reloads of a whole vector
        if (!tag_wait_more(err, t0, spins)) {
          failed = true;
          break;
        }
      }
#pragma unroll
      for (int k = 0; k < SK_PASS; ++k) {
        v[k][0] = act_val(a[k].x);
        v[k][1] = act_val(a[k].y);
        v[k][2] = act_val(a[k].z);
        v[k][3] = act_val(a[k].w);
      }
    }
#pragma unroll
    for (int k = 0; k < SK_PASS; ++k) {
      const int e = 4 * (t + (k0 + k) * SK_THREADS);
      if (k0 + k < ng && e < n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ss = fmaf(v[k][i], v[k][i], ss);
          if (res && e + i >= res_lo && e + i < res_lo + res_n) res[e + i - res_lo] = v[k][i];
        }
        float4 o = make_float4(v[k][0], v[k][1], v[k][2], v[k][3]);
        if (gain) {
          o.x *= g[k].x;
          o.y *= g[k].y;
          o.z *= g[k].z;
          o.w *= g[k].w;
        }
        *reinterpret_cast<float4*>(vin + sk_vin_pos<QW>(e)) = o;
      }
    }
  }
  for (int e = n + 4 * t; e < npad; e += 4 * SK_THREADS)
    *reinterpret_cast<float4*>(vin + sk_vin_pos<QW>(e)) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  return ss;
}

// sum of every thread's x over the workgroup, the same value for all threads
__device__ __forceinline__ float sk_block_sum(float x, float* s_red) {
  x = wave_sum_dpp(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < SK_WAVES; ++w) t += s_red[w];
  return t;
}

// where one op's row results go
struct SkOut {
  uint32_t* y;        // QKV: q|k|v of the layer; O/DN: the new x version; GU: u of the layer
  const float* res;   // O/DN: the workgroup's residual rows of the old x (LDS)
  float* hidden;      // DN: optional copy of x, this layer's row
  float* logits;      // HEAD: optional
  float scale;        // RMSNorm scale of the op's input (1 when there is no norm)
  uint32_t tag;       // act_tag of the step
};

// Row results of one wave, lane-parallel: wave-local row r's dot product is in lane r of y (r < 64) or
// lane r - 64 of y2. Written out once the op's loads are done, so the load loop holds no stores.
template <int KIND, typename Op>
__device__ __forceinline__ void sk_rows_out(float y, float y2, const Op& f, const StepParams& p, const SkRows& R,
                                            const SkOut& out, int wave, int lane, float& best_v, int& best_i) {
  if constexpr (KIND == OP_GU) {
    // gate of output j in lane 2j, its up in lane 2j + 1 (of y, then of y2)
    const float up = __shfl_down(y, 1, 64), up2 = __shfl_down(y2, 1, 64);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lane + 64 * h;
      if ((lane & 1) == 0 && r < f.nrows) {
        const float g = (h ? y2 : y) * out.scale, u = (h ? up2 : up) * out.scale;
        st_act(out.y + R.f.lo + wave + SK_WAVES * (r >> 1), silu_f(g) * u, out.tag);
      }
    }
  } else if constexpr (KIND == OP_HEAD) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lane + 64 * h;
      if (r < f.nrows) {
        const float lg = (h ? y2 : y) * out.scale;
        const int row = R.h.lo + wave + SK_WAVES * r;
        if (out.logits) out.logits[row] = lg;
        if (argmax_better(lg, row, bv, bi)) {
          bv = lg;
          bi = row;
        }
      }
    }
    wave_argmax(bv, bi);
    if (argmax_better(bv, bi, best_v, best_i)) {
      best_v = bv;
      best_i = bi;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = lane + 64 * h;
      if (r < f.nrows) {
        const float v = h ? y2 : y;
        const int q = wave + SK_WAVES * r;
        if constexpr (KIND == OP_QKV) {
          const int idx = q < f.n0 ? R.q.lo + q
                                   : (q < f.n01 ? p.qd + R.k.lo + (q - f.n0) : p.qd + p.kvd + R.v.lo + (q - f.n01));
          st_act(out.y + idx, v * out.scale, out.tag);
        } else {
          const float xn = out.res[q] + v;
          st_act(out.y + R.d.lo + q, xn, out.tag);
          if (KIND == OP_DN && out.hidden) out.hidden[R.d.lo + q] = xn;
        }
      }
    }
  }
}

// One block of SK_R ring slots of op f, starting at slot blk: slot j is read and dotted with the staged
// input, then refilled with slot ib + j of op `is` (when ISSUE). A row's dot product is reduced over the wave
// at its last slot and put into lane r of y (r < 64) or lane r - 64 of y2.
// Dot of 4 int8 codes (one word) with 4 inputs. (Taking the codes as unsigned bytes q + 128, one conversion
// each, and subtracting 128 times the staged input's group sums was measured slower here: 2.78 against
// 2.67 ms for the 8B step; the group sum is one more LDS read in front of every slot's last FMAs.)
__device__ __forceinline__ float sk_dot4_i8(uint32_t w, const float4& x, float acc) {
  acc = fmaf((float)(int8_t)w, x.x, acc);
  acc = fmaf((float)(int8_t)(w >> 8), x.y, acc);
  acc = fmaf((float)(int8_t)(w >> 16), x.z, acc);
  return fmaf((float)(int8_t)(w >> 24), x.w, acc);
}

template <bool ISSUE, bool QW>
__device__ __forceinline__ void sk_block(uint4 (&ring)[SK_R], float (&sring)[SK_R], const SkOp<QW>& f, int blk,
                                         const SkOp<QW>& is, int ib, const float* vl, int wave, int lane, int lane16,
                                         float& acc0, float& acc1, float& y, float& y2) {
  const int mask = (1 << f.sh) - 1;
#pragma unroll
  for (int j = 0; j < SK_R; ++j) {
    const int u = blk + j;
    const int c = u & mask;
    const uint4 r = ring[j];
    if constexpr (QW) {
      // 16 codes times the lane's 16 inputs, then times the group's scale
      const float* xv = vl + c * SK_SEG_Q;
      const float4 x0 = *reinterpret_cast<const float4*>(xv);
      const float4 x1 = *reinterpret_cast<const float4*>(xv + 256);
      const float4 x2 = *reinterpret_cast<const float4*>(xv + 512);
      const float4 x3 = *reinterpret_cast<const float4*>(xv + 768);
      const float d0 = sk_dot4_i8(r.z, x2, sk_dot4_i8(r.x, x0, 0.0f));
      const float d1 = sk_dot4_i8(r.w, x3, sk_dot4_i8(r.y, x1, 0.0f));
      acc0 = fmaf(d0, sring[j], acc0);
      acc1 = fmaf(d1, sring[j], acc1);
    } else {
      const float4 x0 = *reinterpret_cast<const float4*>(vl + c * SK_SEG);
      const float4 x1 = *reinterpret_cast<const float4*>(vl + c * SK_SEG + 256);
      acc0 = fmaf(bf16_lo(r.x), x0.x, acc0);
      acc1 = fmaf(bf16_hi(r.x), x0.y, acc1);
      acc0 = fmaf(bf16_lo(r.y), x0.z, acc0);
      acc1 = fmaf(bf16_hi(r.y), x0.w, acc1);
      acc0 = fmaf(bf16_lo(r.z), x1.x, acc0);
      acc1 = fmaf(bf16_hi(r.z), x1.y, acc1);
      acc0 = fmaf(bf16_lo(r.w), x1.z, acc0);
      acc1 = fmaf(bf16_hi(r.w), x1.w, acc1);
    }
    if constexpr (ISSUE) {
      const float* sa = nullptr;
      ring[j] = gload_stream(sk_addr<QW>(is, ib + j, wave, lane16, &sa));
      if constexpr (QW) sring[j] = gload<float>(sa);
    }
    if (c == mask) {
      const int rr = u >> f.sh;
      const float t = wave_sum_dpp(acc0 + acc1);
      acc0 = acc1 = 0.0f;
      if (rr < f.nrows) {
        y = lane == rr ? t : y;
        y2 = lane == rr - 64 ? t : y2;
      }
    }
  }
}

// Consume the loads of op f from the ring while refilling each slot right after it is read with the slot
// SK_R further on (the last block refills nothing). Nothing but the ring's loads and the LDS reads of the
// input touches memory in the loop, so every slot waits only for its own load.
template <bool QW>
__device__ __forceinline__ void sk_consume(uint4 (&ring)[SK_R], float (&sring)[SK_R], const SkOp<QW>& f, const float* vl,
                                           int wave, int lane, int lane16, float& y, float& y2) {
  float acc0 = 0.0f, acc1 = 0.0f;
  y = 0.0f;
  y2 = 0.0f;
  if (f.npos <= 0) return;
  int blk = 0;
  for (; blk + SK_R < f.npos; blk += SK_R)
    sk_block<true, QW>(ring, sring, f, blk, f, blk + SK_R, vl, wave, lane, lane16, acc0, acc1, y, y2);
  sk_block<false, QW>(ring, sring, f, blk, f, 0, vl, wave, lane, lane16, acc0, acc1, y, y2);
}

// The attention parameters of layer l in the persistent step: (K/V head, context part) items over the context
// 0..pos, parts tagged per layer, q|k|v and the merged output as tagged activations.
template <typename T, int HD>
__device__ __forceinline__ AttnParams sk_attn_params(const StepParams& p, int l, int pos, uint32_t tag) {
  const int ctx = pos + 1;
  const int ch = p.attn_chunk;
  const int n_sub = (ctx + ch - 1) / ch;
  int target = p.nwg / p.Hkv;
  target = target < 1 ? 1 : (target > ATTN_MAX_PARTS ? ATTN_MAX_PARTS : target);
  const int spw = (n_sub + target - 1) / target;
  const StepLayer& Ly = p.layers[l];
  AttnParams ap{};
  ap.H = p.H;
  ap.Hkv = p.Hkv;
  ap.hd = HD;
  ap.kv_is_bf16 = sizeof(T) == 2;
  ap.state = p.state;
  ap.chunk = ch;
  ap.sub_per_wg = spw;
  ap.n_parts = (n_sub + spw - 1) / spw;
  ap.part_tagged = p.attn_part;
  ap.part_tag = tag * STEP_MAX_LAYERS + (uint32_t)l;
  ap.rope_table = p.rope_table;
  ap.rope_layout = p.rope_layout;
  ap.k = static_cast<const char*>(Ly.k) + p.kv_off * (int64_t)sizeof(T);
  ap.v = static_cast<const char*>(Ly.v) + p.kv_off * (int64_t)sizeof(T);
  ap.k_w = static_cast<char*>(Ly.k) + p.kv_off * (int64_t)sizeof(T);
  ap.v_w = static_cast<char*>(Ly.v) + p.kv_off * (int64_t)sizeof(T);
  ap.pg.table = p.kv_table;
  ap.pg.shift = p.kv_shift;
  ap.qkv_tag = p.qkv + (int64_t)l * p.qkv_stride;
  ap.out_tag = p.att + (int64_t)l * p.att_stride;
  ap.tag = p.give_up ? 3u : act_tag(tag - 1u);   // 3: a tag no workgroup writes (tests of the give-up path)
  ap.err = p.err;
  return ap;
}

// RoPE, K/V append and attention of layer l: this workgroup's (K/V head, context part) items, each part's
// (max, sum, output) stored tagged. The tiles live in the dynamic LDS the staged input uses between ops, and
// no weight load is in flight meanwhile, so the registers are the attention's own.
template <typename T, int HD>
__device__ __forceinline__ void sk_attention_items(const StepParams* pp, int l, int pos, uint32_t tag) {
  extern __shared__ uint4 sk_dyn[];
  const StepParams p = *pp;
  const AttnParams ap = sk_attn_params<T, HD>(p, l, pos, tag);
  for (int it = blockIdx.x; it < p.Hkv * ap.n_parts; it += p.nwg)
    attn_block<T, HD, true>(ap, it / ap.n_parts, it % ap.n_parts, 0, sk_dyn);
}

// The merges this workgroup owns (query head hq by workgroup nwg - 1 - hq, from the end, away from the first
// items), which write the tagged attention output. They run before the workgroup's first o weight loads are
// issued: loads return in order, so a merge polling behind those loads would see its parts only once they had
// landed (measured: 3.1725 against 3.179 ms a step with 8 loads a lane in the ring).
template <typename T, int HD>
__device__ __forceinline__ void sk_attention_merges(const StepParams* pp, int l, int pos, uint32_t tag) {
  const StepParams p = *pp;
  const AttnParams ap = sk_attn_params<T, HD>(p, l, pos, tag);
  const int G = p.H / p.Hkv;
  for (int hq = p.nwg - 1 - (int)blockIdx.x; hq < p.H; hq += p.nwg) attn_merge_tagged<HD>(ap, hq / G, hq % G, ap.n_parts);
}

template <typename T, int HD>
constexpr int sk_lds_vecs() {
  return attn_tile_vecs<T, HD>() > STEP_MAX_VIN / 4 ? attn_tile_vecs<T, HD>() : STEP_MAX_VIN / 4;
}

template <typename T, int HD, bool QW>
__global__ __launch_bounds__(SK_THREADS, 1) void step_kernel(const StepParams p) {
  // the staged input vector and the attention tiles are never live together: one region of dynamic LDS
  // (sk_lds_vecs<T, HD>() vectors)
  extern __shared__ uint4 sk_dyn[];
  __shared__ SkLayer s_layers[STEP_MAX_LAYERS];
  __shared__ float s_res[STEP_MAX_RES];      // this workgroup's residual rows of x
  __shared__ float s_red[SK_WAVES];
  __shared__ float s_best_v[SK_WAVES];
  __shared__ int s_best_i[SK_WAVES];
  __shared__ int s_last;
  float* vin = reinterpret_cast<float*>(sk_dyn);

  const int w = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int lane16 = lane * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwg = p.nwg;
  const int L = p.n_layer;
  const int n_ops = 4 * L + 1;
  const int step = p.state->step;
  const int tok = p.state->token;
  const int pos = p.state->pos;
  const uint32_t tag = (uint32_t)step + 1u;      // the attention parts' (with the layer)
  const uint32_t atag = act_tag((uint32_t)step);  // the activations'  
  bool failed = false;

  for (int i = threadIdx.x; i < L; i += SK_THREADS) {
    const StepLayer& s = p.layers[i];
    SkLayer& d = s_layers[i];
#pragma unroll
    for (int j = 0; j < 7; ++j) d.w[j] = s.w[j];
    d.g1 = s.g1;
    d.g2 = s.g2;
    d.k = s.k;
    d.v = s.v;
  }
  SkRows R;
  // Workgroup w runs on XCD w % 8. Where a workgroup's share of gate|up is large (at least 256 KB; 917 KB in the
  // Llama-3-8B shape) the rows of XCD x's workgroups form one contiguous eighth of each matrix: measured 0.35%
  // faster there than workgroup w taking the w-th share, and 1.1% slower in the Qwen3-0.6B shape (48 KB a
  // workgroup), which keeps the w-th share.
  const int64_t gu_share = (int64_t)(p.F / nwg) * 2 * p.d * (QW ? 1 : 2);
  const int wc = nwg % 8 == 0 && gu_share >= (256 << 10) ? (w % 8) * (nwg / 8) + w / 8 : w;
  R.q = sk_range(p.qd, wc, nwg);
  R.k = sk_range(p.kvd, wc, nwg);
  R.v = sk_range(p.kvd, wc, nwg);
  R.d = sk_range(p.d, wc, nwg);
  R.f = sk_range(p.F, wc, nwg);
  R.h = sk_range(p.V, wc, nwg);
  __syncthreads();

#define SK_X(V) (p.x + (int64_t)(V) * p.x_stride)
#define SK_QKV(LL) (p.qkv + (int64_t)(LL) * p.qkv_stride)
#define SK_ATT(LL) (p.att + (int64_t)(LL) * p.att_stride)
#define SK_U(LL) (p.u + (int64_t)(LL) * p.u_stride)


  float best_v = -INFINITY;   // head: this wave's best logit and its row (lane 0)
  int best_i = INT_MAX;

  for (int o = 0; o < n_ops; ++o) {
    const SkOp<QW> f = sk_op<QW>(p, R, s_layers, o, wave);
    // The op's first SK_R loads go out before its input is waited for (for o: after this workgroup's attention
    // items, which need the registers, and after its merges, whose polls would otherwise return only once those
    // loads had landed), so the weights stream while the producers finish.
    if (f.kind == OP_O) {
      sk_attention_items<T, HD>(&p, f.l, pos, tag);
      sk_attention_merges<T, HD>(&p, f.l, pos, tag);
    }
    uint4 ring[SK_R];
    float sring[SK_R];   // int8 packs: each slot's scale
    if (f.npos > 0) {
#pragma unroll
      for (int j = 0; j < SK_R; ++j) {
        const float* sa = nullptr;
        ring[j] = gload_stream(sk_addr<QW>(f, j, wave, lane16, &sa));
        if constexpr (QW) sring[j] = gload<float>(sa);
      }
    }
    // ---- the op's input ----
    SkOut out;
    out.tag = atag;
    out.scale = 1.0f;
    out.res = s_res;
    out.hidden = nullptr;
    out.logits = p.logits;
    const int npad = sk_seg<QW>() << f.sh;
    if (f.kind == OP_O) {
      __syncthreads();
      sk_stage<QW>(SK_ATT(f.l), nullptr, p.qd, npad, atag, nullptr, nullptr, 0, 0, vin, p.err, failed);
      out.y = SK_X(2 * f.l);
    } else if (f.kind == OP_DN) {
      __syncthreads();
      sk_stage<QW>(SK_U(f.l), nullptr, p.F, npad, atag, nullptr, nullptr, 0, 0, vin, p.err, failed);
      out.y = SK_X(2 * f.l + 1);
      out.hidden = p.hidden ? p.hidden + (int64_t)f.l * p.d : nullptr;
    } else {
      // RMSNorm inputs: x before layer l (the embedding row for layer 0), x after layer l's o, final x
      const uint32_t* src = nullptr;
      const bf16_t* emb = nullptr;
      const float* gain;
      if (f.kind == OP_QKV) {
        if (f.l == 0) emb = p.emb + (int64_t)tok * p.d;
        else src = SK_X(2 * f.l - 1);
        gain = s_layers[f.l].g1;
        out.y = SK_QKV(f.l);
      } else if (f.kind == OP_GU) {
        src = SK_X(2 * f.l);
        gain = s_layers[f.l].g2;
        out.y = SK_U(f.l);
      } else {
        src = SK_X(2 * L - 1);
        gain = p.g_final;
        out.y = nullptr;
      }
      __syncthreads();
      const float ss = sk_stage<QW>(src, emb, p.d, npad, atag, gain, f.kind == OP_HEAD ? nullptr : s_res, R.d.lo, R.d.n,
                                vin, p.err, failed);
      out.scale = 1.0f / sqrtf(sk_block_sum(ss, s_red) / (float)p.d + p.eps);
    }
    __syncthreads();

    // ---- the op's loads: dot from the ring, refill the ring ----
    float y, y2;
    sk_consume<QW>(ring, sring, f, vin + lane * 4, wave, lane, lane16, y, y2);
    if (f.npos > 0) {
      switch (f.kind) {
        case OP_QKV: sk_rows_out<OP_QKV>(y, y2, f, p, R, out, wave, lane, best_v, best_i); break;
        case OP_O: sk_rows_out<OP_O>(y, y2, f, p, R, out, wave, lane, best_v, best_i); break;
        case OP_GU: sk_rows_out<OP_GU>(y, y2, f, p, R, out, wave, lane, best_v, best_i); break;
        case OP_DN: sk_rows_out<OP_DN>(y, y2, f, p, R, out, wave, lane, best_v, best_i); break;
        default: sk_rows_out<OP_HEAD>(y, y2, f, p, R, out, wave, lane, best_v, best_i); break;
      }
    }
    // every wave's row results are out before any wave issues the next op's first loads
    __syncthreads();
  }
#undef SK_X
#undef SK_QKV
#undef SK_ATT
#undef SK_U

  // ---- greedy token: each workgroup's best, the last workgroup to finish reduces them ----
  if (lane == 0) {
    s_best_v[wave] = best_v;
    s_best_i[wave] = best_i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = s_best_v[0];
    int ix = s_best_i[0];
    for (int q = 1; q < SK_WAVES; ++q)
      if (argmax_better(s_best_v[q], s_best_i[q], v, ix)) {
        v = s_best_v[q];
        ix = s_best_i[q];
      }
    st_dev(&p.head_val[w], v);
    st_dev(&p.head_idx[w], ix);
    stores_done();
    s_last = (take_ticket(p.head_cnt) == (unsigned)(nwg - 1));
  }
  __syncthreads();
  if (!s_last) return;
  float v = -INFINITY;
  int ix = INT_MAX;
  for (int b = threadIdx.x; b < nwg; b += SK_THREADS) {
    const float bv = ld_dev(&p.head_val[b]);
    const int bi = ld_dev(&p.head_idx[b]);
    if (argmax_better(bv, bi, v, ix)) {
      v = bv;
      ix = bi;
    }
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
      if (argmax_better(s_best_v[q], s_best_i[q], v, ix)) {
        v = s_best_v[q];
        ix = s_best_i[q];
      }
    p.token_out[step] = ix;
    p.state->token = ix;
    p.state->pos = pos + 1;
    p.state->step = step + 1;
    reset_ticket(p.head_cnt);
  }
}

template <typename T, int HD, bool QW>
static const void* step_fn() {
  return reinterpret_cast<const void*>(&step_kernel<T, HD, QW>);
}

// int8 weight packs run with head dims 64, 128 and 256 (the shapes whose widths are whole groups of 128)
static const void* step_kernel_ptr(int kv_is_bf16, int hd, int qw) {
  if (qw) {
    switch (hd) {
      case 64: return kv_is_bf16 ? step_fn<bf16_t, 64, true>() : step_fn<float, 64, true>();
      case 128: return kv_is_bf16 ? step_fn<bf16_t, 128, true>() : step_fn<float, 128, true>();
      case 256: return kv_is_bf16 ? step_fn<bf16_t, 256, true>() : step_fn<float, 256, true>();
    }
    return nullptr;
  }
  switch (hd) {
#define LLMK_SK_CASE(H) \
  case H: return kv_is_bf16 ? step_fn<bf16_t, H, false>() : step_fn<float, H, false>();
    LLMK_SK_CASE(2) LLMK_SK_CASE(4) LLMK_SK_CASE(8) LLMK_SK_CASE(16) LLMK_SK_CASE(32) LLMK_SK_CASE(64)
    LLMK_SK_CASE(128) LLMK_SK_CASE(256)
#undef LLMK_SK_CASE
  }
  return nullptr;
}

static size_t step_lds_bytes(int kv_is_bf16, int hd) {
  switch (hd) {
#define LLMK_SK_CASE(H) \
  case H: return 16 * (size_t)(kv_is_bf16 ? sk_lds_vecs<bf16_t, H>() : sk_lds_vecs<float, H>());
    LLMK_SK_CASE(2) LLMK_SK_CASE(4) LLMK_SK_CASE(8) LLMK_SK_CASE(16) LLMK_SK_CASE(32) LLMK_SK_CASE(64)
    LLMK_SK_CASE(128) LLMK_SK_CASE(256)
#undef LLMK_SK_CASE
  }
  return 0;
}

int step_grid(int kv_is_bf16, int hd, int qw) {
  const void* fn = step_kernel_ptr(kv_is_bf16, hd, qw);
  if (!fn) return 0;
  const size_t lds = step_lds_bytes(kv_is_bf16, hd);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, SK_THREADS, lds) != hipSuccess) return 0;
  return per_cu >= 1 ? cus : 0;
}

hipError_t step_launch(const StepParams& p, int kv_is_bf16, hipStream_t s) {
  const void* fn = step_kernel_ptr(kv_is_bf16, p.hd, p.qw);
  if (!fn || p.nwg < 1) return hipErrorInvalidValue;
  void* args[] = {const_cast<StepParams*>(&p)};
  return hipLaunchKernel(fn, dim3((unsigned)p.nwg), dim3(SK_THREADS), args, step_lds_bytes(kv_is_bf16, p.hd), s);
}

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
