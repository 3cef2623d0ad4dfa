// Device helpers shared by the gfx950 kernels of libllmk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LLMK_WAVE 64

namespace llmk {

typedef uint16_t bf16_t;

// ---- bf16 <-> fp32 ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// ---- typed element access ----------------------------------------------------------------------

template <typename T> __device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T> __device__ __forceinline__ void store_elem(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// A VEC-element slice of a row, loaded as one raw register group (16 B for the vector paths).
template <typename T, int VEC> struct Raw;
template <> struct Raw<bf16_t, 8> { typedef uint4 type; };
template <> struct Raw<float, 4> { typedef uint4 type; };
template <> struct Raw<bf16_t, 1> { typedef uint16_t type; };
template <> struct Raw<float, 1> { typedef float type; };

template <typename T, int VEC>
__device__ __forceinline__ typename Raw<T, VEC>::type load_raw(const T* p) {
  return *reinterpret_cast<const typename Raw<T, VEC>::type*>(p);
}

template <typename T, int VEC>
__device__ __forceinline__ void unpack(const typename Raw<T, VEC>::type& r, float* out);
template <> __device__ __forceinline__ void unpack<bf16_t, 8>(const uint4& r, float* o) {
  o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x); o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
  o[4] = bf16_lo(r.z); o[5] = bf16_hi(r.z); o[6] = bf16_lo(r.w); o[7] = bf16_hi(r.w);
}
template <> __device__ __forceinline__ void unpack<float, 4>(const uint4& r, float* o) {
  o[0] = __uint_as_float(r.x); o[1] = __uint_as_float(r.y); o[2] = __uint_as_float(r.z); o[3] = __uint_as_float(r.w);
}
template <> __device__ __forceinline__ void unpack<bf16_t, 1>(const uint16_t& r, float* o) { o[0] = bf16_to_f32(r); }
template <> __device__ __forceinline__ void unpack<float, 1>(const float& r, float* o) { o[0] = r; }

// ---- wave reductions (wave64) --------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// sum over groups of `width` adjacent lanes (width a power of two <= 64); every lane of a group gets the sum
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum of v over the 64 lanes, returned to every lane, through DPP lane moves (no LDS traffic): inclusive
// prefix sums within each row of 16 lanes (shifts by 1, 2, 4, 8), the row totals carried into the next rows
// by the row broadcasts of lanes 15 and 31, then lane 63's total read out. The order of the additions is
// fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));   // row_shr:1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));   // row_shr:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));   // row_shr:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));   // row_shr:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));   // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Maximum of v over the 64 lanes, returned to every lane, through DPP lane moves (the structure of
// wave_sum_dpp; lanes without a source keep -inf).
__device__ __forceinline__ float wave_max_dpp(float v) {
  const int ninf = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xa, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---- argmax order: NaN above every number (first NaN wins); ties (and +0 == -0) to the lower index --

__device__ __forceinline__ bool argmax_better(float a, int ia, float b, int ib) {
  const bool na = a != a, nb = b != b;
  if (na || nb) {
    if (na && nb) return ia < ib;
    return na;
  }
  if (a > b) return true;
  if (a < b) return false;
  return ia < ib;
}

__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(idx, o, 64);
    if (argmax_better(ov, oi, v, idx)) { v = ov; idx = oi; }
  }
}

// ---- hand-off between workgroups of one launch (split-K partials, argmax and attention partials) ----
// The producer stores with device scope (written through its XCD's L2), waits for its own stores, and
// after a workgroup barrier one thread takes a ticket; the workgroup whose ticket is last reads every
// partial with device-scope loads (served past the non-coherent L2s). No device-wide fence is used: on
// this multi-XCD part a fence writes back and invalidates the whole L2 of the issuing XCD.

__device__ __forceinline__ void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this thread's memory operations (the device-scope stores above all) have completed
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ unsigned take_ticket(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_ticket(unsigned* c) { __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// ---- device-resident decode state ---------------------------------------------------------------

struct DecodeState {
  int32_t token;   // token consumed by the next step
  int32_t pos;     // its position
  int32_t step;    // index of the next step within a multi-step call
  int32_t pad;
};

// Batched decode and prefill chunks: one entry per row (rows <= LLMK_MAX_BATCH_ROWS; a decode batch holds at
// most 64 sequences, a prefill chunk up to 256 rows of one sequence).
constexpr int LLMK_MAX_BATCH_ROWS = 256;
struct BatchState {
  int32_t token[LLMK_MAX_BATCH_ROWS];   // token each row consumes in the next step
  int32_t pos[LLMK_MAX_BATCH_ROWS];     // its position
  int32_t slot[LLMK_MAX_BATCH_ROWS];    // the row's slot in the K/V pool
  int32_t rows;
  int32_t step;                         // index of the next step within a multi-step call
  int32_t pad[2];
};

// hi + lo split of an fp32 value into two bf16 (round to nearest even each): hi + lo carries about 16
// significant bits, the form the batched projections feed to bf16 matrix cores
__device__ __forceinline__ void split_bf16(float v, bf16_t& hi, bf16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Load of a V from global memory through a pointer the compiler cannot see is global (one read from LDS or
// from a table): names the global address space so the load is a global (not a flat) load.
template <typename V>
__device__ __forceinline__ V gload(const void* ptr) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(V) == 16) {
    return __builtin_bit_cast(V, *(const __attribute__((address_space(1))) u32x4*)ptr);
  } else if constexpr (sizeof(V) == 8) {
    return __builtin_bit_cast(V, *(const __attribute__((address_space(1))) u32x2*)ptr);
  } else {
    static_assert(sizeof(V) == 4, "gload: 4, 8 or 16 bytes");
    return __builtin_bit_cast(V, *(const __attribute__((address_space(1))) unsigned*)ptr);
  }
}

// A 16-byte load of data read once and not again soon (weights streamed by a decode step): marked
// non-temporal, so the lines it brings do not displace what the caches hold for other reads (the activations
// workgroups hand each other, the attention's working set). Measured on the persistent 8B step: 3.176 -> 2.940 ms.
__device__ __forceinline__ uint4 gload_stream(const void* ptr) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)ptr));
}

// load_raw for a weight stream: the 16-byte slices non-temporal (gload_stream), narrower ones as load_raw
template <typename T, int VEC>
__device__ __forceinline__ typename Raw<T, VEC>::type load_raw_stream(const T* p) {
  if constexpr (sizeof(typename Raw<T, VEC>::type) == 16) return gload_stream(p);
  else return load_raw<T, VEC>(p);
}

// ---- paged K/V: a slot's positions reach their blocks through its row of the block table ----------------

// The block table as the kernels take it: table == nullptr for contiguous slots.
struct KvPaging {
  const int32_t* table;   // [n_slots][stride] block ids
  int64_t stride;         // entries per slot
  int32_t shift;          // log2 of the positions per block
};

// Cache row of position t of the slot whose table row is `trow` (blocks of 1 << shift positions).
__device__ __forceinline__ int64_t kv_block_row(const int32_t* trow, int shift, int64_t t) {
  return ((int64_t)trow[t >> shift] << shift) | (t & ((int64_t(1) << shift) - 1));
}

}  // namespace llmk
