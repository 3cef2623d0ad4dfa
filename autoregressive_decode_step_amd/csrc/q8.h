// Launch interface of the int8 weight kernels (host side of libllmk).
//
// A q8 pack holds a [rows][K] matrix (output-major) quantized per group of Q8_GROUP consecutive inputs of
// a row: rows*K int8 codes, row-major, then rows*(K/Q8_GROUP) fp32 scales, row-major; element (r, k) is
// codes[r*K + k] * scales[r*(K/Q8_GROUP) + k/Q8_GROUP].
#pragma once

#include "kernels.h"

namespace llmk {

constexpr int Q8_GROUP = 128;

inline int64_t q8_pack_bytes(int64_t rows, int64_t K) { return rows * K + 4 * rows * (K / Q8_GROUP); }

// Quantize a [rows][K] matrix (fp32, or bf16 when w_is_bf16) into a q8 pack. K % Q8_GROUP == 0.
hipError_t q8_quantize_launch(const void* w, int w_is_bf16, int64_t rows, int64_t K, void* pack, hipStream_t s);

// Row-dot GEMV over q8 packs, with the modes of rowdot_launch (w0/w1/w2 are packs; the embedding row of
// in_is_w and base_is_w is bf16). Fills kw/np/r/rows_per_block/n_blocks; -1 if K does not fit.
int rowdot_q8_plan(RowdotParams& p, int mode);
hipError_t rowdot_q8_launch(const RowdotParams& p, int mode, hipStream_t s);

// After a greedy head: token_out[state->step] = *tok; the state consumes it at the next position.
hipError_t state_advance_launch(DecodeState* st, const int32_t* tok, int32_t* token_out, hipStream_t s);

}  // namespace llmk
