// Launch interface of the sampled decode loop's glue kernels (host side of libllmk).
#pragma once

#include "kernels.h"

namespace llmk {

// dst[0] = draws[st->step - 1]: the uniform of the step whose head has just advanced the state.
hipError_t draw_pick_launch(const DecodeState* st, const float* draws, float* dst, hipStream_t s);
// The sampled token *tok replaces the greedy one: tokens_out[st->step - 1] = *tok, and the state consumes it
// at the next position.
hipError_t sampled_token_launch(DecodeState* st, const int32_t* tok, int32_t* tokens_out, hipStream_t s);

}  // namespace llmk
