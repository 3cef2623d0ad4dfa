// Paged K/V pool for gfx950: the host block manager (block table mirror, reference counts, copy-on-write,
// refusal when full, admission) and the two kernels it drives, plus the paged flat append.
// ("Inside the engine", "3. The K/V cache and the block store": the cache is paged in fixed blocks that
// sequences forked from a common prefix share by reference count, copied on write; a full pool refuses the
// append. "2. The scheduler: continuous batching", "Admission": free blocks must cover the uncached suffix
// plus decode headroom.)
#include <string.h>

#include <unordered_map>
#include <vector>

#include "kvpages.h"

namespace llmk {

constexpr int PG_THREADS = 256;

// ---- kernels ---------------------------------------------------------------------------------------------

__global__ void table_set_kernel(int32_t* table, const TableEdits e) {
  const int i = threadIdx.x;
  if (i < e.n) table[e.idx[i]] = e.val[i];
}

hipError_t table_set_launch(int32_t* table, const TableEdits& e, hipStream_t s) {
  static_assert(TABLE_EDITS <= 64, "one wave writes the edits");
  hipLaunchKernelGGL(table_set_kernel, dim3(1), dim3(64), 0, s, table, e);
  return hipGetLastError();
}

template <typename T>
__global__ void kv_append_paged_kernel(T* cache, const int32_t* trow, int shift, int64_t row_elems, int64_t first,
                                       const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = first + i;
    const int64_t pos = f / row_elems;
    store_elem<T>(cache, kv_block_row(trow, shift, pos) * row_elems + (f - pos * row_elems), src[i]);
  }
}

hipError_t kv_append_paged_launch(void* cache, int is_bf16, const int32_t* trow, int shift, int64_t row_elems,
                                  int64_t first, const float* src, int64_t n, hipStream_t s) {
  const int64_t want = (n + PG_THREADS - 1) / PG_THREADS;
  const dim3 grid((unsigned)(want < 4096 ? want : 4096));
  if (is_bf16)
    hipLaunchKernelGGL(kv_append_paged_kernel<bf16_t>, grid, dim3(PG_THREADS), 0, s, static_cast<bf16_t*>(cache), trow,
                       shift, row_elems, first, src, n);
  else
    hipLaunchKernelGGL(kv_append_paged_kernel<float>, grid, dim3(PG_THREADS), 0, s, static_cast<float*>(cache), trow,
                       shift, row_elems, first, src, n);
  return hipGetLastError();
}

// ---- host block manager ----------------------------------------------------------------------------------

namespace {

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int shift_of(int64_t bt) {
  int k = 0;
  while ((int64_t(1) << k) < bt) ++k;
  return k;
}

// Enqueues the table writes in launches of TABLE_EDITS.
hipError_t flush_edits(int32_t* table, const std::vector<std::pair<int64_t, int32_t>>& edits, hipStream_t s) {
  hipError_t e = hipSuccess;
  for (size_t i0 = 0; i0 < edits.size() && e == hipSuccess; i0 += TABLE_EDITS) {
    TableEdits te;
    memset(&te, 0, sizeof(te));
    te.n = (int32_t)std::min<size_t>(TABLE_EDITS, edits.size() - i0);
    for (int32_t k = 0; k < te.n; ++k) {
      te.idx[k] = edits[i0 + k].first;
      te.val[k] = edits[i0 + k].second;
    }
    e = table_set_launch(table, te, s);
  }
  return e;
}

}  // namespace

int32_t pages_check(const llmk_kv_pool* p) {
  const llmk_kv_pages* g = p->pages;
  if (!g->table || !g->table_h || !g->refcount_h) return LLMK_INVALID_ARGUMENT;
  if (!pow2(g->block_tokens) || g->block_tokens < 64 || g->block_tokens > 65536) return LLMK_INVALID_ARGUMENT;
  if (g->max_blocks != (p->capacity + g->block_tokens - 1) / g->block_tokens) return LLMK_INVALID_ARGUMENT;
  if (g->n_blocks < 1) return LLMK_EMPTY_DIMENSION;
  if (g->n_blocks > LLMK_MAX_DIM || p->n_slots * g->max_blocks > LLMK_MAX_DIM) return LLMK_DIMENSION_TOO_LARGE;
  return LLMK_OK;
}

int pages_shift(const llmk_kv_pool* p) { return p->pages ? shift_of(p->pages->block_tokens) : 0; }

int64_t pool_rows(const llmk_kv_pool* p) {
  return p->pages ? p->pages->n_blocks * p->pages->block_tokens : p->n_slots * p->capacity;
}

float* pool_scales(const llmk_kv_pool* p, void* buf) {
  return reinterpret_cast<float*>(static_cast<char*>(buf) + pool_rows(p) * p->n_kv * p->head_dim);
}

KvPaging pages_view(const llmk_kv_pool* p) {
  KvPaging v{};
  if (p->pages) {
    v.table = p->pages->table;
    v.stride = p->pages->max_blocks;
    v.shift = shift_of(p->pages->block_tokens);
  }
  return v;
}

const int32_t* pages_slot_row(const llmk_kv_pool* p, int64_t slot) {
  return p->pages ? p->pages->table + slot * p->pages->max_blocks : nullptr;
}

int64_t pages_row(const llmk_kv_pool* p, int64_t slot, int64_t pos) {
  const llmk_kv_pages* g = p->pages;
  const int32_t b = g->table_h[slot * g->max_blocks + pos / g->block_tokens];
  return b < 0 ? -1 : (int64_t)b * g->block_tokens + pos % g->block_tokens;
}

int32_t pages_reserve(llmk_kv_pool* p, const KvReserve* req, int64_t n, hipStream_t s) {
  llmk_kv_pages* g = p->pages;
  const int64_t BT = g->block_tokens, MB = g->max_blocks;
  for (int64_t r = 0; r < n; ++r)
    if (req[r].end > p->capacity) return LLMK_CACHE_CAPACITY_EXCEEDED;
  // pass 1: the blocks the requests take, with the reference drops of copies made earlier in this call
  std::unordered_map<int32_t, int32_t> dropped;
  int64_t need = 0;
  for (int64_t r = 0; r < n; ++r) {
    if (req[r].end <= req[r].begin) continue;
    for (int64_t j = req[r].begin / BT; j <= (req[r].end - 1) / BT; ++j) {
      const int32_t b = g->table_h[req[r].slot * MB + j];
      if (b < 0) {
        ++need;
      } else if (g->refcount_h[b] - dropped[b] > 1) {
        ++need;
        ++dropped[b];
      }
    }
  }
  if (need == 0) return LLMK_OK;
  if (need > g->n_free) return LLMK_CACHE_CAPACITY_EXCEEDED;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return LLMK_DEVICE_ERROR;
  if (cap != hipStreamCaptureStatusNone) return LLMK_INVALID_ARGUMENT;
  // the `need` lowest-numbered free blocks, in order
  std::vector<int32_t> fresh;
  fresh.reserve((size_t)need);
  for (int64_t b = 0; b < g->n_blocks && (int64_t)fresh.size() < need; ++b)
    if (g->refcount_h[b] == 0) fresh.push_back((int32_t)b);
  if ((int64_t)fresh.size() < need) return LLMK_DEVICE_ERROR;   // n_free disagrees with the refcounts
  // pass 2: assign them (the same walk as pass 1)
  std::vector<std::pair<int64_t, int32_t>> edits;
  std::vector<std::pair<int32_t, int32_t>> copies;   // (from, to)
  size_t k = 0;
  for (int64_t r = 0; r < n; ++r) {
    if (req[r].end <= req[r].begin) continue;
    for (int64_t j = req[r].begin / BT; j <= (req[r].end - 1) / BT; ++j) {
      const int64_t idx = req[r].slot * MB + j;
      const int32_t b = g->table_h[idx];
      if (b >= 0 && g->refcount_h[b] == 1) continue;
      const int32_t nb = fresh[k++];
      if (b >= 0) {
        --g->refcount_h[b];
        copies.emplace_back(b, nb);
      }
      g->refcount_h[nb] = 1;
      g->table_h[idx] = nb;
      edits.emplace_back(idx, nb);
    }
  }
  g->n_free -= need;
  // copy-on-write: the whole block, every layer, K and V (an int8 pool's scales too)
  hipError_t e = hipSuccess;
  const bool q8 = p->dtype == LLMK_Q8;
  const int64_t bytes = BT * p->n_kv * p->head_dim * (q8 ? 1 : p->dtype == LLMK_BF16 ? 2 : 4);
  const int64_t sbytes = BT * p->n_kv * 4;
  for (const auto& c : copies)
    for (int64_t l = 0; l < p->n_layer && e == hipSuccess; ++l)
      for (int w = 0; w < 2 && e == hipSuccess; ++w) {
        char* buf = static_cast<char*>(w == 0 ? p->k[l] : p->v[l]);
        e = hipMemcpyAsync(buf + (int64_t)c.second * bytes, buf + (int64_t)c.first * bytes, (size_t)bytes,
                           hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && q8) {
          char* sc = reinterpret_cast<char*>(pool_scales(p, buf));
          e = hipMemcpyAsync(sc + (int64_t)c.second * sbytes, sc + (int64_t)c.first * sbytes, (size_t)sbytes,
                             hipMemcpyDeviceToDevice, s);
        }
      }
  if (e == hipSuccess) e = flush_edits(g->table, edits, s);
  return e == hipSuccess ? LLMK_OK : LLMK_DEVICE_ERROR;
}

}  // namespace llmk

// =========================================================================================================
// C ABI: fork, release, admission, reserve
// =========================================================================================================

using namespace llmk;

namespace {

// A pool's own fields and its pages, which must be set.
int32_t paged_pool_check(const llmk_kv_pool* p) {
  if (!p) return LLMK_INVALID_ARGUMENT;
  const int32_t st = pool_fields_check(p);
  if (st != LLMK_OK) return st;
  return p->pages ? LLMK_OK : LLMK_INVALID_ARGUMENT;
}

void set_records(llmk_kv_pool* p, int64_t slot, int64_t n_pos) {
  p->slot_len_h[slot] = n_pos;
  const int64_t row = p->n_kv * p->head_dim;
  for (int64_t l = 0; l < p->n_layer; ++l) {
    if (p->len_k_h) p->len_k_h[l * p->n_slots + slot] = n_pos * row;
    if (p->len_v_h) p->len_v_h[l * p->n_slots + slot] = n_pos * row;
  }
}

}  // namespace

extern "C" {

int32_t llmk_kv_reserve(llmk_kv_pool* pool, int64_t slot, int64_t pos_begin, int64_t pos_end, void* stream) {
  int32_t st = paged_pool_check(pool);
  if (st != LLMK_OK) return st;
  if (pos_begin < 0 || pos_end <= pos_begin) return LLMK_EMPTY_DIMENSION;
  if (pos_end > LLMK_MAX_DIM) return LLMK_DIMENSION_TOO_LARGE;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  const KvReserve r{slot, pos_begin, pos_end};
  return pages_reserve(pool, &r, 1, static_cast<hipStream_t>(stream));
}

int32_t llmk_kv_fork(llmk_kv_pool* pool, int64_t src, int64_t dst, int64_t n_pos, void* stream) {
  int32_t st = paged_pool_check(pool);
  if (st != LLMK_OK) return st;
  if (src == dst) return LLMK_INVALID_ARGUMENT;
  if (n_pos < 1) return LLMK_EMPTY_DIMENSION;
  if (n_pos > LLMK_MAX_DIM) return LLMK_DIMENSION_TOO_LARGE;
  if (src < 0 || src >= pool->n_slots || dst < 0 || dst >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  llmk_kv_pages* g = pool->pages;
  const int64_t MB = g->max_blocks, nb = (n_pos + g->block_tokens - 1) / g->block_tokens;
  if (n_pos > pool->slot_len_h[src] || pool->slot_len_h[dst] != 0) return LLMK_CACHE_LENGTH_MISMATCH;
  for (int64_t j = 0; j < MB; ++j)
    if (g->table_h[dst * MB + j] >= 0) return LLMK_CACHE_LENGTH_MISMATCH;
  for (int64_t j = 0; j < nb; ++j)
    if (g->table_h[src * MB + j] < 0) return LLMK_CACHE_LENGTH_MISMATCH;   // src's positions without a block
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess) return LLMK_DEVICE_ERROR;
  if (cap != hipStreamCaptureStatusNone) return LLMK_INVALID_ARGUMENT;
  std::vector<std::pair<int64_t, int32_t>> edits;
  for (int64_t j = 0; j < nb; ++j) {
    const int32_t b = g->table_h[src * MB + j];
    g->table_h[dst * MB + j] = b;
    ++g->refcount_h[b];
    edits.emplace_back(dst * MB + j, b);
  }
  set_records(pool, dst, n_pos);
  return flush_edits(g->table, edits, static_cast<hipStream_t>(stream)) == hipSuccess ? LLMK_OK : LLMK_DEVICE_ERROR;
}

int32_t llmk_kv_release(llmk_kv_pool* pool, int64_t slot) {
  int32_t st = paged_pool_check(pool);
  if (st != LLMK_OK) return st;
  if (slot < 0 || slot >= pool->n_slots) return LLMK_SLOT_OUT_OF_RANGE;
  llmk_kv_pages* g = pool->pages;
  for (int64_t j = 0; j < g->max_blocks; ++j) {
    int32_t& b = g->table_h[slot * g->max_blocks + j];
    if (b >= 0 && --g->refcount_h[b] == 0) ++g->n_free;
    b = -1;
  }
  set_records(pool, slot, 0);
  return LLMK_OK;
}

int32_t llmk_kv_admit(const llmk_kv_pool* pool, int64_t n_uncached, int32_t* admit_h) {
  if (!admit_h) return LLMK_INVALID_ARGUMENT;
  int32_t st = paged_pool_check(pool);
  if (st != LLMK_OK) return st;
  if (n_uncached < 0) return LLMK_EMPTY_DIMENSION;
  if (n_uncached > LLMK_MAX_DIM) return LLMK_DIMENSION_TOO_LARGE;
  const int64_t bt = pool->pages->block_tokens;
  *admit_h = pool->pages->n_free >= (n_uncached + bt - 1) / bt + 1 ? 1 : 0;
  return LLMK_OK;
}

}  // extern "C"
