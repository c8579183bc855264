// Internal declarations of the verify-set selector.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace va {

// Longest score row the selector handles.  A row whose candidate list
// cannot be resolved from the filter's output is resolved by one workgroup
// that re-reads the row in 32768-token segments on every radix pass; the
// limit bounds that time.
constexpr int32_t kSelectSegTokens = 32768;
constexpr int32_t kSelectMaxL = 24 * kSelectSegTokens;

size_t select_ws_bytes(int32_t B, int32_t L);

hipError_t launch_select(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                         int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                         void* ws, hipStream_t stream);

}  // namespace va
