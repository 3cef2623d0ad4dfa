// The sampling exit of a decode step for gfx950: one draw per row of logits.
//
// Stages in the sequence of the "decode-ops" page ("Method"): temperature, the k-largest cut, the
// probability-mass cut, then the caller's uniform draw chooses among what is left by its cumulative
// distribution; candidates rank by logit, equal logits lower index first. A candidate stays while the weight
// ranked ahead of it is under p (the shortest prefix whose weight reaches p: the HuggingFace warper rule the
// page names), and the token is the first staying candidate where the running share of the staying weight
// passes u.
// Temperature 0 is the greedy exit: the lowest index holding the maximum.
//
// A positive temperature does not change the order of the logits, so the survivors are chosen on the raw
// logits and the temperature enters only their weights exp((z - z_max) / T), taken in fp64. Every logit
// becomes an order-preserving 32-bit key; an entry (~key << 32 | index) then sorts ascending in exactly
// the survivor order, and the key gives the value back.
//
// No float atomics anywhere, so a row and a draw always give the same token. Three forms, by row length and k:
//   wave slices (the usual one): a row is cut into G slices of 1,024 (else 2,048) logits with G * k <=
//     SAMPLE_MERGE_MAX. One wave per slice holds the slice's keys in registers (16 or 32 a lane) and emits the
//     slice's own top-k (ties to the lower index) to the workspace: every survivor of the row is among them.
//     One workgroup per row then keeps the candidates at or above the k-th largest slice maximum (a floor for
//     the row's k-th largest) and ranks them in LDS, or, when that leaves too many, selects the row's top-k
//     from all G * k candidates (8 a thread, in registers); then it draws.
//   block slices (larger k): the same with slices of 16,384 logits, one 1024-thread workgroup each.
//   wide (rows too long for either): one workgroup per row selects straight from the logits with a radix
//     select over LDS histograms (four passes of 8-bit digits, sixteen histogram copies so that lanes hitting
//     one bin rarely meet).
// The register selection builds the k-th largest key bit by bit from the top: a bit stays set while at least
// k keys are at or above the prefix, each count a ballot per register. When the count meets k exactly the
// survivors are known early; otherwise ties at the k-th key are cut the same way on their index bits.
#include <algorithm>

#include "kernels.h"
#include "loop.h"

namespace llmk {

constexpr int SM_THREADS = 1024;
constexpr int SM_WAVES = SM_THREADS / 64;
constexpr int SM_BINS = 256;
constexpr int SM_COPIES = 16;              // lane l counts into histogram copy l % 16
constexpr int SM_STRIDE = SM_BINS + 1;     // the pad puts the copies of one bin in different LDS banks
constexpr int SAMPLE_MERGE_R = 8;                                // candidates per merge thread
constexpr int SAMPLE_MERGE_MAX = SM_THREADS * SAMPLE_MERGE_R;    // candidates one row's merge holds
constexpr int SW_WAVES = 4;                                      // wave slices per workgroup (16 or 32 keys a lane)
constexpr int SM_TAU_SLICES = 256;                               // slice maxima the merge's bound takes
constexpr int SB_R = 16;                                         // keys per thread of a block slice
constexpr int SB_CHUNK = SM_THREADS * SB_R;                      // logits per block slice
constexpr int SM_INDEX_BITS = 24;                                // indices below 2^24 (rows of at most 2^24)
static_assert(SAMPLE_MAX_K <= SM_THREADS, "one survivor per thread in the scans");
static_assert(SAMPLE_MAX_K <= SAMPLE_MERGE_MAX, "one slice's survivors fit the merge");
static_assert(SM_BINS == 4 * 64, "one wave scans the bins, four per lane");

// a logit as the sampler orders it: NaN is -inf, and -0 is +0 (the two compare equal, so ties decide)
__device__ __forceinline__ float sm_val(float v) {
  if (v != v) return -INFINITY;
  return v == 0.0f ? 0.0f : v;
}

// an order-preserving key: larger value, larger key
__device__ __forceinline__ uint32_t sm_key(float v) {
  const uint32_t b = __float_as_uint(sm_val(v));
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float sm_key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

__device__ __forceinline__ unsigned long long sm_entry(uint32_t key, int64_t i) {
  return ((unsigned long long)(~key) << 32) | (unsigned long long)i;   // ascending = the survivor order
}
__device__ __forceinline__ uint32_t sm_entry_key(unsigned long long e) { return ~(uint32_t)(e >> 32); }
__device__ __forceinline__ int32_t sm_entry_index(unsigned long long e) { return (int32_t)(e & 0xFFFFFFFFull); }

// exclusive prefix over the block of one value per thread (a fixed order), and the total
template <typename V>
__device__ __forceinline__ V sm_block_scan(V v, V* s_w, V& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  V incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const V o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  V before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < SM_WAVES; ++w) {
    before += w < wave ? s_w[w] : V(0);
    all += s_w[w];
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

struct SmSelectLds {
  unsigned hist[SM_COPIES * SM_STRIDE];
  unsigned bin[SM_BINS];
  unsigned wu[SM_WAVES];
  uint32_t prefix;
  unsigned rem;      // survivors not yet above the selected prefix
  unsigned eq;       // keys equal to the selected prefix
  unsigned count;    // survivors emitted
};

// Emits the top `kth` of the `cnt` keys key_at(0..cnt) in any order, each as emit(slot, entry) with the
// slots 0..kth-1 used once: every key above the kth largest, then the lowest-index ties at it. Entries carry
// the index base + i. Block-wide: every thread calls it.
template <typename KeyAt, typename Emit>
__device__ void sm_emit_top(KeyAt key_at, int64_t cnt, int64_t base, unsigned kth, SmSelectLds& L, Emit emit) {
  const int t = threadIdx.x;
  unsigned* const my_hist = L.hist + (t & (SM_COPIES - 1)) * SM_STRIDE;
  if (t == 0) {
    L.prefix = 0u;
    L.rem = kth;
    L.count = 0u;
  }
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = t; b < SM_COPIES * SM_STRIDE; b += SM_THREADS) L.hist[b] = 0u;
    __syncthreads();
    const uint32_t prefix = L.prefix;
    const unsigned rem = L.rem;
    for (int64_t i = t; i < cnt; i += SM_THREADS) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&my_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t < SM_BINS) {
      unsigned c = 0u;
#pragma unroll
      for (int r = 0; r < SM_COPIES; ++r) c += L.hist[r * SM_STRIDE + t];
      L.bin[t] = c;
    }
    __syncthreads();
    if (t < 64) {
      // lane t holds bins 4t..4t+3; the bin whose count from above first reaches rem holds the kth largest
      unsigned h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = L.bin[4 * t + j];
      const unsigned mine = h[0] + h[1] + h[2] + h[3];
      unsigned suf = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = __shfl_down(suf, off, 64);
        if (t + off < 64) suf += o;
      }
      unsigned above = suf - mine;   // keys in the bins of the lanes above
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < rem && rem <= above + h[j]) {
          L.prefix = prefix | ((uint32_t)(4 * t + j) << shift);
          L.rem = rem - above;
          L.eq = h[j];
        }
        above += h[j];
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tk = L.prefix;
  const unsigned take = L.rem;          // ties at tk among the top kth
  const bool all_ties = take == L.eq;   // block-uniform
  for (int64_t i = t; i < cnt; i += SM_THREADS) {
    const uint32_t key = key_at(i);
    if (key > tk || (all_ties && key == tk)) emit(atomicAdd(&L.count, 1u), sm_entry(key, base + i));
  }
  if (!all_ties) {
    // only the lowest-index ties survive: each thread scans a contiguous range, so the block scan of the
    // per-thread tie counts ranks them in index order
    const int64_t chunk = (cnt + SM_THREADS - 1) / SM_THREADS;
    const int64_t lo = min(cnt, (int64_t)t * chunk), hi = min(cnt, lo + chunk);
    unsigned ties = 0u;
    for (int64_t i = lo; i < hi; ++i) ties += key_at(i) == tk ? 1u : 0u;
    unsigned tie_total;
    unsigned rank = sm_block_scan<unsigned>(ties, L.wu, tie_total);
    for (int64_t i = lo; i < hi && rank < take; ++i) {
      if (key_at(i) == tk) {
        emit(atomicAdd(&L.count, 1u), sm_entry(tk, base + i));
        ++rank;
      }
    }
  }
  __syncthreads();
}

struct SmFinishLds {
  unsigned wu[SM_WAVES];
  double wd[SM_WAVES];
  int32_t cut;
};

// The draw over the k survivors s[0..k), already in order: weights, the top-p cut, the inverse CDF.
// Block-wide; thread 0 writes the token.
__device__ void sm_finish(const unsigned long long* s, int k, float temperature, float top_p, float u,
                          int32_t* token, SmFinishLds& F) {
  const int t = threadIdx.x;
  const float v0 = sm_key_value(sm_entry_key(s[0]));
  if (k == 1 || !(v0 > -INFINITY && v0 < INFINITY)) {
    // greedy, a single survivor, or no survivor with a finite weight: the first survivor
    if (t == 0) *token = sm_entry_index(s[0]);
    return;
  }
  double w = 0.0;
  if (t < k) {
    const float v = sm_key_value(sm_entry_key(s[t]));
    w = exp(((double)v - (double)v0) / (double)temperature);   // -inf survivors weigh 0
  }
  double W;
  const double before = sm_block_scan<double>(w, F.wd, W);
  const double incl = before + w;
  // kept: the survivors whose mass before them is below p (the first one always)
  unsigned kept_total;
  sm_block_scan<unsigned>((t < k && (t == 0 || before < (double)top_p * W)) ? 1u : 0u, F.wu, kept_total);
  const int kept = (int)kept_total;
  if (t == kept - 1) F.wd[0] = incl;   // the kept mass
  __syncthreads();
  const double Wk = F.wd[0];
  u = u >= 0.0f ? u : 0.0f;            // a NaN or negative draw counts as 0
  const double target = (double)u * Wk;
  // the token: the first kept survivor whose cumulative mass exceeds the target; past the rounded total,
  // the last kept survivor with mass
  unsigned below;
  sm_block_scan<unsigned>((t < kept && incl <= target) ? 1u : 0u, F.wu, below);
  if (t == 0) F.cut = -1;
  __syncthreads();
  if (t < kept && w > 0.0) atomicMax(&F.cut, t);
  __syncthreads();
  if (t == 0) {
    const int j = (int)below < kept ? (int)below : max(F.cut, 0);
    *token = sm_entry_index(s[j]);
  }
}

// Sorts the k distinct entries in[0..k) ascending into out (each thread < k counts the entries below its own).
__device__ void sm_rank_sort(const unsigned long long* in, unsigned long long* out, int k) {
  const int t = threadIdx.x;
  if (t < k) {
    const unsigned long long e = in[t];
    int r = 0;
    for (int i = 0; i < k; ++i) r += in[i] < e ? 1 : 0;
    out[r] = e;
  }
  __syncthreads();
}

// ---- selection over keys held in registers by a group: one wave, or the whole 1024-thread block ----
// Key j of thread i of the group is at position j * THREADS + i.

// key[j] of thread i of the group: the logit at position j * THREADS + i of x[0..len), or 0 past the end
template <int R, int THREADS>
__device__ __forceinline__ void sm_load_keys(const float* x, int64_t len, int i, uint32_t (&key)[R]) {
  float v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = x[min((int64_t)j * THREADS + i, len - 1)];   // in bounds, len >= 1
  // the loads are all issued before any value is used (the compiler would otherwise move each load into
  // a branch of its own and wait for it there)
#pragma unroll
  for (int j = 0; j < R; ++j) asm volatile("" : "+v"(v[j]));
#pragma unroll
  for (int j = 0; j < R; ++j) key[j] = (int64_t)j * THREADS + i < len ? sm_key(v[j]) : 0u;
}

template <int THREADS>
__device__ __forceinline__ unsigned grp_sum(unsigned wave_count, unsigned* s_red, int& parity) {
  static_assert(THREADS == 64 || THREADS == SM_THREADS, "a wave or the block");
  if constexpr (THREADS == 64) {
    return wave_count;
  } else {
    // two buffers in turn: a buffer is rewritten only after every wave has passed the barrier that follows
    // the last reads of it
    unsigned* const buf = s_red + parity * SM_WAVES;
    parity ^= 1;
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = wave_count;
    __syncthreads();
    unsigned sum = 0u;
#pragma unroll
    for (int w = 0; w < SM_WAVES; ++w) sum += buf[w];
    return sum;
  }
}

template <int THREADS, int R, typename Pred>
__device__ __forceinline__ unsigned grp_count(Pred pred, unsigned* s_red, int& parity) {
  unsigned c = 0u;
#pragma unroll
  for (int j = 0; j < R; ++j) c += (unsigned)__popcll(__ballot(pred(j)));
  return grp_sum<THREADS>(c, s_red, parity);
}

// the survivors of a selection: every key above `key`, and the keys equal to it whose index is below `iend`
struct GrpCut {
  uint32_t key;
  uint32_t iend;
  __device__ __forceinline__ bool keeps(uint32_t k, uint32_t i) const { return k > key || (k == key && i < iend); }
};

// The top kth of the group's keys, ties to the lower index; at least kth keys must be real (padding keys are 0,
// below every real key). Group-wide.
template <int THREADS, int R, typename IndexAt>
__device__ GrpCut grp_select(const uint32_t (&key)[R], IndexAt index_at, unsigned kth, unsigned* s_red) {
  int parity = 0;
  uint32_t T = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = T | (1u << b);
    const unsigned c = grp_count<THREADS, R>([&](int j) { return key[j] >= t; }, s_red, parity);
    if (c == kth) return {t - 1u, 0u};   // exactly kth keys at or above t
    if (c > kth) T = t;
  }
  // T is the kth largest key: the keys above it survive, and the lowest-index `take` of the ties at it
  const unsigned gt = T == 0xFFFFFFFFu ? 0u : grp_count<THREADS, R>([&](int j) { return key[j] > T; }, s_red, parity);
  const unsigned take = kth - gt;
  const unsigned eq = grp_count<THREADS, R>([&](int j) { return key[j] == T; }, s_red, parity);
  if (eq == take) return {T, 0xFFFFFFFFu};
  uint32_t X = 0u;   // the take-th smallest tie index, built the same way
  for (int b = SM_INDEX_BITS - 1; b >= 0; --b) {
    const uint32_t t = X | (1u << b);
    const unsigned c =
        grp_count<THREADS, R>([&](int j) { return key[j] == T && index_at(j) < t; }, s_red, parity);
    if (c < take) X = t;
  }
  return {T, X + 1u};
}

// wide form: one workgroup per row selects straight from the logits
__global__ __launch_bounds__(SM_THREADS) void sample_wide_kernel(const float* logits, int64_t n, float temperature,
                                                                 int32_t k, float top_p, const float* draw,
                                                                 int32_t* token) {
  __shared__ SmSelectLds L;
  __shared__ SmFinishLds F;
  __shared__ unsigned long long s_list[SAMPLE_MAX_K];
  __shared__ unsigned long long s_sorted[SAMPLE_MAX_K];
  const int64_t row = blockIdx.x;
  const float* x = logits + row * n;
  sm_emit_top([&](int64_t i) { return sm_key(x[i]); }, n, 0, (unsigned)k, L,
              [&](unsigned slot, unsigned long long e) { s_list[slot] = e; });
  sm_rank_sort(s_list, s_sorted, k);
  sm_finish(s_sorted, k, temperature, top_p, draw[row], token + row, F);
}

// wave slices, step 1: wave w of workgroup (row r, y) takes slice g = y * SW_WAVES + w (64 R logits, R a lane)
// and writes its top-k to cand[r][g][0..k) in index order; the slots past the slice's length hold entries that
// sort last
template <int R>
__global__ __launch_bounds__(64 * SW_WAVES) void sample_wave_slice_kernel(const float* logits, int64_t n,
                                                                          int32_t slices, int32_t k,
                                                                          unsigned long long* cand, uint32_t* smax) {
  constexpr int CHUNK = 64 * R;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.y * SW_WAVES + (threadIdx.x >> 6);
  if (g >= slices) return;   // wave-uniform; the kernel has no barrier
  const int64_t row = blockIdx.x;
  const int64_t lo = (int64_t)g * CHUNK, len = min((int64_t)CHUNK, n - lo);
  const float* x = logits + row * n + lo;
  unsigned long long* out = cand + (row * slices + g) * (int64_t)k;
  uint32_t key[R];
  sm_load_keys<R, 64>(x, len, lane, key);
  const unsigned kl = (unsigned)min((int64_t)k, len);
  for (int64_t j = (int64_t)kl + lane; j < k; j += 64) out[j] = ~0ull;
  uint32_t mx = 0u;   // the slice's largest key
#pragma unroll
  for (int j = 0; j < R; ++j) mx = max(mx, key[j]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if (lane == 0) smax[row * slices + g] = mx;
  auto index_at = [&](int j) { return (uint32_t)(lo + (int64_t)j * 64 + lane); };
  const GrpCut cut = grp_select<64, R>(key, index_at, kl, nullptr);
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned slot = 0u;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const bool keep = cut.keeps(key[j], index_at(j));
    const unsigned long long m = __ballot(keep);
    if (keep) out[slot + (unsigned)__popcll(m & below)] = sm_entry(key[j], index_at(j));
    slot += (unsigned)__popcll(m);
  }
}

// block slices, step 1: workgroup (row r, slice g) writes its slice's top-k to cand[r][g][0..k) in any order;
// the slots past the slice's length hold entries that sort last
__global__ __launch_bounds__(SM_THREADS) void sample_block_slice_kernel(const float* logits, int64_t n,
                                                                        int32_t k, unsigned long long* cand,
                                                                        uint32_t* smax) {
  __shared__ unsigned s_red[2 * SM_WAVES];
  __shared__ unsigned s_n;
  __shared__ uint32_t s_max;
  const int t = threadIdx.x;
  const int g = blockIdx.y, slices = gridDim.y;
  const int64_t row = blockIdx.x;
  const int64_t lo = (int64_t)g * SB_CHUNK, len = min((int64_t)SB_CHUNK, n - lo);
  const float* x = logits + row * n + lo;
  unsigned long long* out = cand + (row * slices + g) * (int64_t)k;
  uint32_t key[SB_R];
  sm_load_keys<SB_R, SM_THREADS>(x, len, t, key);
  const unsigned kl = (unsigned)min((int64_t)k, len);
  for (int64_t j = (int64_t)kl + t; j < k; j += SM_THREADS) out[j] = ~0ull;
  if (t == 0) {
    s_n = 0u;
    s_max = 0u;
  }
  __syncthreads();
  uint32_t mx = 0u;   // the slice's largest key
#pragma unroll
  for (int j = 0; j < SB_R; ++j) mx = max(mx, key[j]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if ((t & 63) == 0) atomicMax(&s_max, mx);
  __syncthreads();
  if (t == 0) smax[row * slices + g] = s_max;
  auto index_at = [&](int j) { return (uint32_t)(lo + (int64_t)j * SM_THREADS + t); };
  const GrpCut cut = grp_select<SM_THREADS, SB_R>(key, index_at, kl, s_red);   // its barriers order s_n
#pragma unroll
  for (int j = 0; j < SB_R; ++j)
    if (cut.keeps(key[j], index_at(j))) out[atomicAdd(&s_n, 1u)] = sm_entry(key[j], index_at(j));
}

// step 2 of either slice form: one workgroup per row selects the top k of the n_cand candidates (k per slice),
// ranks them and draws.
// With at least k slices, the k-th largest of the slices' maxima is a floor for the row's k-th largest key
// (those k maxima are k distinct logits), so every survivor is among the candidates at or above it. When they
// are few (1,024 at most, the usual case) each ranks itself against the others in LDS; otherwise the whole
// candidate set goes through the bit-by-bit selection.
__global__ __launch_bounds__(SM_THREADS) void sample_merge_kernel(const unsigned long long* cand,
                                                                  const uint32_t* smax, int32_t n_cand, int32_t k,
                                                                  float temperature, float top_p, const float* draw,
                                                                  int32_t* token) {
  __shared__ unsigned s_red[2 * SM_WAVES];
  __shared__ unsigned s_n;
  __shared__ uint32_t s_tau;
  __shared__ SmFinishLds F;
  __shared__ unsigned long long s_list[SAMPLE_MAX_K];
  __shared__ unsigned long long s_sorted[SAMPLE_MAX_K];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const unsigned long long* c = cand + row * n_cand;
  unsigned long long e[SAMPLE_MERGE_R];
  uint32_t key[SAMPLE_MERGE_R];
#pragma unroll
  for (int j = 0; j < SAMPLE_MERGE_R; ++j) e[j] = c[min(j * SM_THREADS + t, n_cand - 1)];
#pragma unroll
  for (int j = 0; j < SAMPLE_MERGE_R; ++j) asm volatile("" : "+v"(e[j]));   // every load issued before any use
#pragma unroll
  for (int j = 0; j < SAMPLE_MERGE_R; ++j) {
    e[j] = j * SM_THREADS + t < n_cand ? e[j] : ~0ull;
    key[j] = sm_entry_key(e[j]);   // the entries that sort last have key 0
  }
  const int slices = n_cand / k;
  if (slices >= k && slices <= SM_TAU_SLICES) {   // block-uniform
    if (t == 0) s_n = 0u;
    if (t < 64) {   // one wave: the k-th largest slice maximum, or a value with exactly k maxima at or above it
      const uint32_t* sm = smax + row * slices;
      uint32_t mk[SM_TAU_SLICES / 64];
#pragma unroll
      for (int r = 0; r < SM_TAU_SLICES / 64; ++r) mk[r] = r * 64 + t < slices ? sm[r * 64 + t] : 0u;
      const GrpCut c = grp_select<64, SM_TAU_SLICES / 64>(mk, [&](int r) { return (uint32_t)(r * 64 + t); },
                                                          (unsigned)k, nullptr);
      if (t == 0) s_tau = c.iend == 0u ? c.key + 1u : c.key;
    }
    __syncthreads();
    const uint32_t tau = s_tau;
#pragma unroll
    for (int j = 0; j < SAMPLE_MERGE_R; ++j) {
      if (j * SM_THREADS + t < n_cand && key[j] >= tau) {
        const unsigned slot = atomicAdd(&s_n, 1u);
        if (slot < SAMPLE_MAX_K) s_list[slot] = e[j];
      }
    }
    __syncthreads();
    const unsigned m = s_n;
    if (m <= (unsigned)SAMPLE_MAX_K) {
      if (t < (int)m) {
        const unsigned long long mine = s_list[t];
        int r = 0;
        for (unsigned i = 0; i < m; ++i) r += s_list[i] < mine ? 1 : 0;
        if (r < k) s_sorted[r] = mine;
      }
      __syncthreads();
      sm_finish(s_sorted, k, temperature, top_p, draw[row], token + row, F);
      return;
    }
    __syncthreads();   // too many at the floor: the full selection below
  }
  if (t == 0) s_n = 0u;
  auto index_at = [&](int j) { return (uint32_t)sm_entry_index(e[j]); };
  const GrpCut cut = grp_select<SM_THREADS, SAMPLE_MERGE_R>(key, index_at, (unsigned)k, s_red);
#pragma unroll
  for (int j = 0; j < SAMPLE_MERGE_R; ++j)
    if (cut.keeps(key[j], index_at(j))) s_list[atomicAdd(&s_n, 1u)] = e[j];
  __syncthreads();
  sm_rank_sort(s_list, s_sorted, k);
  sm_finish(s_sorted, k, temperature, top_p, draw[row], token + row, F);
}

SamplePlan sample_plan(int64_t n, int32_t k) {
  for (int64_t chunk : {64 * 16, 64 * 32}) {   // wave slices: 16, else 32 keys a lane
    const int64_t gw = (n + chunk - 1) / chunk;
    if (gw > 1 && gw * k <= SAMPLE_MERGE_MAX) return {SAMPLE_WAVE_SLICES, (int)gw, chunk};
  }
  const int64_t gb = (n + SB_CHUNK - 1) / SB_CHUNK;
  if (gb > 1 && gb * k <= SAMPLE_MERGE_MAX) return {SAMPLE_BLOCK_SLICES, (int)gb, SB_CHUNK};
  return {SAMPLE_WIDE, 1, n};
}

// workspace of the slice forms: the candidates [rows][slices][k], then the slice maxima [rows][slices]
int64_t sample_workspace_bytes(int64_t rows, int64_t n, int32_t k) {
  const SamplePlan p = sample_plan(n, k);
  if (p.form == SAMPLE_WIDE) return 0;
  return rows * p.slices * ((int64_t)k * (int64_t)sizeof(unsigned long long) + (int64_t)sizeof(uint32_t));
}

hipError_t sample_launch(const float* logits, int64_t rows, int64_t n, float temperature, int32_t k, float top_p,
                         const float* draw, int32_t* token, void* ws, hipStream_t s) {
  const SamplePlan p = sample_plan(n, k);
  if (p.form == SAMPLE_WIDE) {
    hipLaunchKernelGGL(sample_wide_kernel, dim3((unsigned)rows), dim3(SM_THREADS), 0, s, logits, n, temperature, k,
                       top_p, draw, token);
    return hipGetLastError();
  }
  auto* cand = static_cast<unsigned long long*>(ws);
  uint32_t* smax = reinterpret_cast<uint32_t*>(cand + rows * p.slices * (int64_t)k);
  if (p.form == SAMPLE_WAVE_SLICES) {
    const dim3 grid((unsigned)rows, (unsigned)((p.slices + SW_WAVES - 1) / SW_WAVES));
    if (p.chunk == 64 * 16)
      hipLaunchKernelGGL(sample_wave_slice_kernel<16>, grid, dim3(64 * SW_WAVES), 0, s, logits, n, (int32_t)p.slices,
                         k, cand, smax);
    else
      hipLaunchKernelGGL(sample_wave_slice_kernel<32>, grid, dim3(64 * SW_WAVES), 0, s, logits, n, (int32_t)p.slices,
                         k, cand, smax);
  } else {
    hipLaunchKernelGGL(sample_block_slice_kernel, dim3((unsigned)rows, (unsigned)p.slices), dim3(SM_THREADS), 0, s,
                       logits, n, k, cand, smax);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_merge_kernel, dim3((unsigned)rows), dim3(SM_THREADS), 0, s, cand, smax,
                     (int32_t)(p.slices * k), k, temperature, top_p, draw, token);
  return hipGetLastError();
}

// ---- glue of the sampled decode loop (one thread each; the state lives on the device) -------------------

__global__ void draw_pick_kernel(const DecodeState* st, const float* draws, float* dst) {
  if (threadIdx.x == 0) dst[0] = draws[st->step - 1];
}

__global__ void sampled_token_kernel(DecodeState* st, const int32_t* tok, int32_t* tokens_out) {
  if (threadIdx.x != 0) return;
  const int32_t t = tok[0];
  tokens_out[st->step - 1] = t;
  st->token = t;
}

hipError_t draw_pick_launch(const DecodeState* st, const float* draws, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(draw_pick_kernel, dim3(1), dim3(64), 0, s, st, draws, dst);
  return hipGetLastError();
}

hipError_t sampled_token_launch(DecodeState* st, const int32_t* tok, int32_t* tokens_out, hipStream_t s) {
  hipLaunchKernelGGL(sampled_token_kernel, dim3(1), dim3(64), 0, s, st, tok, tokens_out);
  return hipGetLastError();
}

}  // namespace llmk
