// Causal attention of a prefill chunk on gfx950 matrix cores.
//
// The rows of a prompt chunk are consecutive positions of one sequence, so they attend over the same cached
// keys and values ("Inside the engine", "1. CausalLM: the forward path": prefill is a chunk of rows through
// the batched routes, with flash attention over the sequence's K/V). A workgroup takes 64 query vectors of one
// K/V head (64 / G rows of the chunk times the G query heads sharing that K/V head) and one part of the context
// (up to 256 positions), stages each 64-position K tile and V tile in LDS once for all 64 queries, and keeps a
// running softmax per query (max, sum, unnormalised output), as the split-context decode attention does for one
// query. Scores S = Q K^T and the output O += P V run on v_mfma_f32_16x16x32_bf16: q, the probabilities and
// fp32 K/V are carried as bf16 hi + lo (products of the parts taken separately into fp32), bf16 K/V are exact.
// Each wave owns 16 of the queries. Keys past a query's own position are masked (causal). The parts of one
// query are combined afterwards with their log-sum-exp weights, in part order.
//
// Layouts of one 16 x 16 x 32 product: the A operand gives lane l row l % 16 and eight consecutive k of group
// l / 16, the B operand likewise for its 16 columns, and the result gives lane l rows 4 (l / 16) .. + 3 at
// column l % 16. Q and K are staged [vector or position][dim]; V is staged transposed, [dim][position], and
// the probabilities go through LDS [query][position], so every operand read is one 16-byte LDS load.
#include <algorithm>

#include "kernels.h"

namespace llmk {

typedef __bf16 fa_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float fa_f32x4_t __attribute__((ext_vector_type(4)));

constexpr int FA_THREADS = 256;
constexpr int FA_QV = 64;      // query vectors per workgroup
constexpr int FA_CH = 64;      // positions per K/V tile
constexpr int FA_HD = 128;     // head dim this kernel takes
constexpr int FA_QS = FA_HD + 8;     // LDS row stride (bf16) of Q and K
constexpr int FA_VS = FA_CH + 8;     // LDS row stride (bf16) of V^T and P

__device__ __forceinline__ fa_f32x4_t fa_mfma(const uint4& a, const uint4& b, const fa_f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fa_bf16x8_t, a),
                                                 __builtin_bit_cast(fa_bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 fa_ld(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// max / sum over the 16 lanes that share l / 16 (lanes l ^ 1, 2, 4, 8)
__device__ __forceinline__ float fa_max16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float fa_sum16(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__global__ __launch_bounds__(FA_THREADS) void fattn_kernel(const FattnParams p) {
  constexpr bool LO = sizeof(T) == 4;   // fp32 K/V carry a lo part
  __shared__ __align__(16) bf16_t s_qh[FA_QV][FA_QS];
  __shared__ __align__(16) bf16_t s_ql[FA_QV][FA_QS];
  __shared__ __align__(16) bf16_t s_kh[FA_CH][FA_QS];
  __shared__ __align__(16) bf16_t s_kl[LO ? FA_CH : 1][LO ? FA_QS : 8];
  __shared__ __align__(16) bf16_t s_vh[FA_HD][FA_VS];
  __shared__ __align__(16) bf16_t s_vl[LO ? FA_HD : 1][LO ? FA_VS : 8];
  __shared__ __align__(16) bf16_t s_ph[4][16][FA_VS];
  __shared__ __align__(16) bf16_t s_pl[4][16][FA_VS];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int G = p.H / p.Hkv, QR = FA_QV / G;     // query heads per K/V head, chunk rows per workgroup
  const int part = blockIdx.x, kvh = blockIdx.z;
  const int r0 = blockIdx.y * QR;
  const int r_end = min(p.rows, r0 + QR);
  const int qpos_max = p.st->pos[r_end - 1];
  const int tb = part * p.span;
  if (tb > qpos_max) return;                     // no query of this tile reaches this part
  const int te = min(tb + p.span, qpos_max + 1);
  const int64_t rstride = (int64_t)p.Hkv * FA_HD;
  // the chunk's slot: its region (contiguous pool) or its row of the block table (paged pool; a tile of FA_CH
  // positions sits in one block)
  const int32_t* const trow = p.pg.table ? p.pg.table + (int64_t)p.st->slot[r0] * p.pg.stride : nullptr;
  const int64_t rbase = (trow ? 0 : (int64_t)p.st->slot[r0] * p.slot_elems) + (int64_t)kvh * FA_HD;
  const T* K = static_cast<const T*>(p.k) + rbase;
  const T* V = static_cast<const T*>(p.v) + rbase;
  const float scale = 1.0f / sqrtf((float)FA_HD);

  // q of the 64 vectors (vector v: chunk row r0 + v / G, query head kvh * G + v % G), rotated by the row's
  // position, as hi + lo; vectors past the chunk are zero
  constexpr int HALF = FA_HD / 2;
  static_assert(FA_QV * 4 == FA_THREADS && HALF % 4 == 0, "four threads per query vector");
  {
    // thread t takes vector t / 4 and rotation pairs 16 (t % 4) .. + 15; every load is issued before any use
    // (rows past the chunk read the last row and are zeroed)
    constexpr int NJ = HALF / 4;
    const int v = t >> 2, j0 = (t & 3) * NJ;
    const int row = r0 + v / G;
    const int rowc = min(row, r_end - 1);
    const float* q = p.qkv + (int64_t)rowc * p.qkv_stride + (int64_t)(kvh * G + v % G) * FA_HD;
    const float* tab = p.rope_table + ((int64_t)p.st->pos[rowc] * HALF + j0) * 2;
    float a[NJ], b[NJ], cs[NJ], sn[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = j0 + jj;
      a[jj] = q[p.rope_layout == 0 ? j : 2 * j];
      b[jj] = q[p.rope_layout == 0 ? j + HALF : 2 * j + 1];
      cs[jj] = tab[2 * jj];
      sn[jj] = tab[2 * jj + 1];
    }
    const float keep = row < r_end ? 1.0f : 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = j0 + jj;
      const int ia = p.rope_layout == 0 ? j : 2 * j;
      const int ib = p.rope_layout == 0 ? j + HALF : 2 * j + 1;
      bf16_t h, l;
      split_bf16(keep * (a[jj] * cs[jj] - b[jj] * sn[jj]), h, l);
      s_qh[v][ia] = h;
      s_ql[v][ia] = l;
      split_bf16(keep * (a[jj] * sn[jj] + b[jj] * cs[jj]), h, l);
      s_qh[v][ib] = h;
      s_ql[v][ib] = l;
    }
  }

  // this lane's four query rows (of the wave's 16): vector 16 w + 4 (l / 16) + e, its position
  int qpos[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int v = wave * 16 + (lane >> 4) * 4 + e;
    const int row = r0 + v / G;
    qpos[e] = row < r_end ? p.st->pos[row] : -1;   // -1: no key is visible, the vector is padding
  }
  float m_run[4], l_run[4];
  fa_f32x4_t o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m_run[e] = -INFINITY;
    l_run[e] = 0.0f;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = fa_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // K/V tile staging: lane l of wave w takes position l of the tile and dims 8 (w + 4 j) .. + 7 for j = 0..3, so
  // the transposed V writes of a wave fill contiguous LDS rows. The next tile's loads are issued as soon as
  // the current tile is in LDS and complete while it is multiplied. Positions past te repeat te - 1 (masked).
  constexpr int NG = FA_CH * FA_HD / 8 / FA_THREADS;       // 8-element groups per thread and tile
  constexpr int VPG = sizeof(T) / 2;                        // 16-byte loads per group
  uint4 kr[NG * VPG], vr[NG * VPG];
  auto load_tile = [&](int t0) {
    const int64_t pos = (trow ? kv_block_row(trow, p.pg.shift, t0) - t0 : 0) + min(t0 + lane, te - 1);
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int c = (wave + 4 * j) * 8;
#pragma unroll
      for (int u = 0; u < VPG; ++u) {
        kr[j * VPG + u] = *reinterpret_cast<const uint4*>(K + pos * rstride + c + u * (8 / VPG));
        vr[j * VPG + u] = *reinterpret_cast<const uint4*>(V + pos * rstride + c + u * (8 / VPG));
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int c = (wave + 4 * j) * 8;
      // pairs of bf16 (element 2e in the low half): the hi parts, and the lo parts of an fp32 cache
      uint32_t kh[4], kl[4], vh[4], vl[4];
      if constexpr (LO) {
        const uint32_t kw[8] = {kr[2 * j].x, kr[2 * j].y, kr[2 * j].z, kr[2 * j].w,
                                kr[2 * j + 1].x, kr[2 * j + 1].y, kr[2 * j + 1].z, kr[2 * j + 1].w};
        const uint32_t vw[8] = {vr[2 * j].x, vr[2 * j].y, vr[2 * j].z, vr[2 * j].w,
                                vr[2 * j + 1].x, vr[2 * j + 1].y, vr[2 * j + 1].z, vr[2 * j + 1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16_t h0, l0, h1, l1;
          split_bf16(__uint_as_float(kw[2 * e]), h0, l0);
          split_bf16(__uint_as_float(kw[2 * e + 1]), h1, l1);
          kh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          kl[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
          split_bf16(__uint_as_float(vw[2 * e]), h0, l0);
          split_bf16(__uint_as_float(vw[2 * e + 1]), h1, l1);
          vh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          vl[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        *reinterpret_cast<uint4*>(&s_kl[lane][c]) = make_uint4(kl[0], kl[1], kl[2], kl[3]);
      } else {
        kh[0] = kr[j].x, kh[1] = kr[j].y, kh[2] = kr[j].z, kh[3] = kr[j].w;
        vh[0] = vr[j].x, vh[1] = vr[j].y, vh[2] = vr[j].z, vh[3] = vr[j].w;
      }
      *reinterpret_cast<uint4*>(&s_kh[lane][c]) = make_uint4(kh[0], kh[1], kh[2], kh[3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_vh[c + 2 * e][lane] = (bf16_t)(vh[e] & 0xFFFFu);
        s_vh[c + 2 * e + 1][lane] = (bf16_t)(vh[e] >> 16);
        if constexpr (LO) {
          s_vl[c + 2 * e][lane] = (bf16_t)(vl[e] & 0xFFFFu);
          s_vl[c + 2 * e + 1][lane] = (bf16_t)(vl[e] >> 16);
        }
      }
    }
  };

  const int orow = lane & 15, ok8 = (lane >> 4) * 8;
  load_tile(tb);
  for (int t0 = tb; t0 < te; t0 += FA_CH) {
    __syncthreads();   // q staged (first tile) / the previous tile's K, V and P fully read
    store_tile();
    if (t0 + FA_CH < te) load_tile(t0 + FA_CH);
    __syncthreads();

    // S = Q K^T for the wave's 16 queries x 64 positions (4 column tiles of 16)
    fa_f32x4_t s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = fa_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < FA_HD / 32; ++ks) {
      const uint4 qh = fa_ld(&s_qh[wave * 16 + orow][ks * 32 + ok8]);
      const uint4 ql = fa_ld(&s_ql[wave * 16 + orow][ks * 32 + ok8]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 kh = fa_ld(&s_kh[j * 16 + orow][ks * 32 + ok8]);
        s[j] = fa_mfma(qh, kh, s[j]);
        s[j] = fa_mfma(ql, kh, s[j]);
        if constexpr (LO) s[j] = fa_mfma(qh, fa_ld(&s_kl[j * 16 + orow][ks * 32 + ok8]), s[j]);
      }
    }

    // online softmax per query row e (the row's 64 scores lie on the 16 lanes of this lane's group x 4 tiles)
    float alpha[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float mt = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kpos = t0 + j * 16 + orow;
        float v = s[j][e] * scale;
        if (kpos > qpos[e] || kpos >= te) v = -INFINITY;
        s[j][e] = v;
        mt = fmaxf(mt, v);
      }
      mt = fa_max16(mt);
      const float m_new = fmaxf(m_run[e], mt);
      alpha[e] = m_new == -INFINITY ? 1.0f : expf(m_run[e] - m_new);
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = s[j][e] == -INFINITY ? 0.0f : expf(s[j][e] - m_new);
        s[j][e] = pr;
        ls += pr;
      }
      l_run[e] = l_run[e] * alpha[e] + fa_sum16(ls);
      m_run[e] = m_new;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[d][e] *= alpha[e];

    // P to LDS [query][position] as hi + lo (this wave's region)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16_t h, l;
        split_bf16(s[j][e], h, l);
        s_ph[wave][(lane >> 4) * 4 + e][j * 16 + orow] = h;
        s_pl[wave][(lane >> 4) * 4 + e][j * 16 + orow] = l;
      }
    __syncthreads();   // P stored before it is read in the operand layout

    // O += P V: 8 column tiles of 16 dims, 2 steps of 32 positions
#pragma unroll
    for (int ks = 0; ks < FA_CH / 32; ++ks) {
      const uint4 ph = fa_ld(&s_ph[wave][orow][ks * 32 + ok8]);
      const uint4 pl = fa_ld(&s_pl[wave][orow][ks * 32 + ok8]);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint4 vh = fa_ld(&s_vh[d * 16 + orow][ks * 32 + ok8]);
        o[d] = fa_mfma(ph, vh, o[d]);
        o[d] = fa_mfma(pl, vh, o[d]);
        if constexpr (LO) o[d] = fa_mfma(ph, fa_ld(&s_vl[d * 16 + orow][ks * 32 + ok8]), o[d]);
      }
    }
  }

  // this part's record per query: unnormalised output, max, sum
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int v = wave * 16 + (lane >> 4) * 4 + e;
    const int row = r0 + v / G;
    if (row >= r_end) continue;
    const int h = kvh * G + v % G;
    float* rec = p.part + (((int64_t)row * p.H + h) * p.n_parts + part) * (FA_HD + 2);
#pragma unroll
    for (int d = 0; d < 8; ++d) rec[d * 16 + orow] = o[d][e];
    if (orow == 0) {
      rec[FA_HD] = m_run[e];
      rec[FA_HD + 1] = l_run[e];
    }
  }
}

// combine the parts 0 .. pos / span of (row, head) with their log-sum-exp weights, in part order, eight parts'
// records loaded at a time (a running maximum rescales what is summed so far), and write hi + lo
constexpr int FA_MERGE_PARTS = 32;   // parts a merge takes (contexts up to 8,192 positions)
constexpr int FA_MERGE_GROUP = 8;
__global__ __launch_bounds__(FA_HD) void fattn_merge_kernel(const FattnParams p) {
  const int row = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const int np = p.st->pos[row] / p.span + 1;
  const float* rec = p.part + ((int64_t)row * p.H + h) * p.n_parts * (FA_HD + 2);
  float m = -INFINITY, L = 0.0f, acc = 0.0f;
  for (int q0 = 0; q0 < np; q0 += FA_MERGE_GROUP) {
    float mq[FA_MERGE_GROUP], lq[FA_MERGE_GROUP], oq[FA_MERGE_GROUP];
#pragma unroll
    for (int j = 0; j < FA_MERGE_GROUP; ++j) {   // parts past np read part q0 again and weigh nothing
      const float* r = rec + (q0 + j < np ? q0 + j : q0) * (FA_HD + 2);
      mq[j] = r[FA_HD];
      lq[j] = r[FA_HD + 1];
      oq[j] = r[i];
    }
    float mg = m;
#pragma unroll
    for (int j = 0; j < FA_MERGE_GROUP; ++j)
      if (q0 + j < np) mg = fmaxf(mg, mq[j]);
    const float sc = m == -INFINITY ? 0.0f : expf(m - mg);
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < FA_MERGE_GROUP; ++j) {
      const float w = (q0 + j >= np || mq[j] == -INFINITY) ? 0.0f : expf(mq[j] - mg);
      L += w * lq[j];
      acc += w * oq[j];
    }
    m = mg;
  }
  bf16_t hi, lo;
  split_bf16(acc / L, hi, lo);
  const int64_t off = (int64_t)row * p.H * FA_HD + (int64_t)h * FA_HD + i;
  p.out_hi[off] = hi;
  p.out_lo[off] = lo;
}

int64_t fattn_parts(int64_t max_ctx) { return (max_ctx + FA_SPAN - 1) / FA_SPAN; }

bool fattn_supported(int64_t H, int64_t Hkv, int64_t hd, int64_t max_ctx) {
  return hd == FA_HD && H % Hkv == 0 && FA_QV % (H / Hkv) == 0 && fattn_parts(max_ctx) <= FA_MERGE_PARTS;
}

hipError_t fattn_launch(const FattnParams& p, int64_t max_ctx, hipStream_t s) {
  if (!fattn_supported(p.H, p.Hkv, FA_HD, max_ctx) || p.span != FA_SPAN || fattn_parts(max_ctx) > p.n_parts)
    return hipErrorInvalidValue;
  const int G = p.H / p.Hkv, QR = FA_QV / G;
  const dim3 grid((unsigned)fattn_parts(max_ctx), (unsigned)((p.rows + QR - 1) / QR), (unsigned)p.Hkv);
  if (p.kv_is_bf16)
    hipLaunchKernelGGL(fattn_kernel<bf16_t>, grid, dim3(FA_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(fattn_kernel<float>, grid, dim3(FA_THREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fattn_merge_kernel, dim3((unsigned)p.rows, (unsigned)p.H), dim3(FA_HD), 0, s, p);
  return hipGetLastError();
}

}  // namespace llmk
