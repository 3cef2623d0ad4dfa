// Paged K/V pool: the host block manager over a pool's block table ("Inside the engine", "3. The K/V cache
// and the block store": fixed blocks shared by reference count with copy-on-write, a full pool refuses;
// "2. The scheduler: continuous batching", "Admission").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llmk.h"
#include "kernels.h"

namespace llmk {

// The pages fields of a pool (pages non-null): 578 / 561 / 564 as llmk_kv_pool_init documents them.
int32_t pages_check(const llmk_kv_pool* p);

// A pool descriptor's own fields (p non-null; no config to compare with) and, when set, its pages:
// llmk_kv_pool_init's codes.
int32_t pool_fields_check(const llmk_kv_pool* p);

// Positions [begin, end) of one slot to be made writable.
struct KvReserve {
  int64_t slot, begin, end;
};

// Reserves every request (distinct slots) or none: fresh blocks for entries of -1, private copies of shared
// blocks, lowest-numbered free blocks first, in request order and then block order. The block copies and
// table writes go on `s`. LLMK_OK, 571 (capacity or free blocks; nothing changed), 578 (capturing with
// device work to do; nothing changed) or 579.
int32_t pages_reserve(llmk_kv_pool* p, const KvReserve* req, int64_t n, hipStream_t s);

// Cache row of (slot, pos) from the host mirror of the table, or -1 when its block is not reserved.
int64_t pages_row(const llmk_kv_pool* p, int64_t slot, int64_t pos);

// The kernels' view of the pool's table: nullptr table for a contiguous pool.
KvPaging pages_view(const llmk_kv_pool* p);

// A slot's device table row (nullptr for a contiguous pool).
const int32_t* pages_slot_row(const llmk_kv_pool* p, int64_t slot);

// log2 of the block size.
int pages_shift(const llmk_kv_pool* p);

// Cache rows of each layer buffer: n_slots * capacity, or n_blocks * block_tokens for a paged pool.
int64_t pool_rows(const llmk_kv_pool* p);

// An int8 pool's layer buffer holds the codes of every cache row, then one fp32 scale per (row, K/V head):
// the scales of buffer `buf`.
float* pool_scales(const llmk_kv_pool* p, void* buf);

}  // namespace llmk
