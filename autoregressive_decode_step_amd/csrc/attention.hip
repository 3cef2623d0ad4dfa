// Split-context grouped-query decode attention for gfx950: the kernel and its plan (the workgroup body
// is in attn_block.h).
#include <algorithm>

#include "attn_block.h"

namespace llmk {

template <typename T, int HD>
__global__ __launch_bounds__(ATTN_THREADS) void attn_kernel(const AttnParams p) {
  __shared__ uint4 tiles[attn_tile_vecs<T, HD>()];
  attn_block<T, HD>(p, blockIdx.y, blockIdx.x, blockIdx.z, tiles);
}

static int tile_rows(int kv_is_bf16, int hd) {   // an int8 cache's tiles are staged as bf16
  const int row_bytes = ((hd * (kv_is_bf16 ? 2 : 4)) + 15) / 16 * 16;
  return attn_tile_rows(row_bytes);
}

void attn_plan(AttnParams& p, int64_t max_ctx, int64_t min_tiles_per_part) {
  p.chunk = tile_rows(p.kv_is_bf16 || p.kv_q8, p.hd);
  const int64_t n_sub = (max_ctx + p.chunk - 1) / p.chunk;
  int64_t target = (n_sub + min_tiles_per_part - 1) / std::max<int64_t>(1, min_tiles_per_part);
  if (target < 1) target = 1;
  if (target > ATTN_MAX_PARTS) target = ATTN_MAX_PARTS;
  int64_t spw = (n_sub + target - 1) / target;
  if (spw < 1) spw = 1;
  p.sub_per_wg = (int32_t)spw;
  p.n_parts = (int32_t)((n_sub + spw - 1) / spw);
}

template <typename T, int HD>
static hipError_t attn_one(const AttnParams& p, hipStream_t s) {
  const unsigned rows = p.bstate ? (unsigned)p.rows : 1u;
  hipLaunchKernelGGL((attn_kernel<T, HD>), dim3((unsigned)p.n_parts, (unsigned)p.Hkv, rows), dim3(ATTN_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_hd(const AttnParams& p, hipStream_t s) {
  switch (p.hd) {
    case 2: return attn_one<T, 2>(p, s);
    case 4: return attn_one<T, 4>(p, s);
    case 8: return attn_one<T, 8>(p, s);
    case 16: return attn_one<T, 16>(p, s);
    case 32: return attn_one<T, 32>(p, s);
    case 64: return attn_one<T, 64>(p, s);
    case 128: return attn_one<T, 128>(p, s);
    case 256: return attn_one<T, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

static hipError_t attn_hd_q8(const AttnParams& p, hipStream_t s) {
  switch (p.hd) {   // int8 rows are whole 16-code loads
    case 16: return attn_one<int8_t, 16>(p, s);
    case 32: return attn_one<int8_t, 32>(p, s);
    case 64: return attn_one<int8_t, 64>(p, s);
    case 128: return attn_one<int8_t, 128>(p, s);
    case 256: return attn_one<int8_t, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t attn_launch(const AttnParams& p, hipStream_t s) {
  if (p.H / p.Hkv > 8 || p.H % p.Hkv != 0) return hipErrorInvalidValue;
  if (p.kv_q8) return attn_hd_q8(p, s);
  return p.kv_is_bf16 ? attn_hd<bf16_t>(p, s) : attn_hd<float>(p, s);
}

}  // namespace llmk
