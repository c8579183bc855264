// Internal declarations of the verify-set selector.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace va {

// Longest score row the selector handles.  The kernel keeps one mark word
// per thread and 32768-token segment in LDS (4 KiB per segment) beside about
// 48 KiB of histograms; 24 segments keep the total within a CU's 160 KiB.
constexpr int32_t kSelectSegTokens = 32768;
constexpr int32_t kSelectMaxL = 24 * kSelectSegTokens;

size_t select_ws_bytes(int32_t B, int32_t L);

hipError_t launch_select(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                         int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                         void* ws, hipStream_t stream);

}  // namespace va
