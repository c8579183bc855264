// Verify-set selection for sparse verification (Dustin, "Aggregazione
// Ibrida dell'Attenzione"): keep the attention-sink prefix and the local
// window, take the top-m tokens by draft-lookahead score, then fill the rest
// of the budget with the best remaining tokens by target-historical score.
//
// One workgroup of 1024 threads per sequence.  Each tier is an exact top-r
// over the contiguous candidate range [lo, hi) between sink and window:
//   * scores become order-preserving 32-bit keys (NaN lowest, -0 == +0);
//   * four 8-bit radix passes (LDS histograms, integer atomics, so the counts
//     do not depend on thread order) find the key T of the r-th best token
//     and the number of tokens strictly above it;
//   * one ordered pass marks every token above T and the first tokens equal
//     to T in index order (a block-wide prefix count), which is the
//     lower-index tie rule.
// The marks live in a bitmap in LDS; a final ordered compaction writes the
// union of sink, window and both tiers as an ascending index list.

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "va_select.h"

namespace va {
namespace {

constexpr int kST = 1024;
constexpr int kSWaves = kST / 64;

struct SelParams {
  const float* ds;
  const float* ts;
  int32_t* out;
  int64_t ld;
  int L, sink, window, top_m, budget, k_out;
};

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;               // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;        // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `pred` over the workgroup in thread order; sets
// *total.  Uses wsum[kSWaves]; contains two barriers.
__device__ inline int block_prefix_count(bool pred, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(pred);
  const uint64_t below = lane ? (bal & (~0ull >> (64 - lane))) : 0ull;
  const int in_wave = __popcll(below);
  if (lane == 0) wsum[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSWaves; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

__device__ inline bool marked(const uint32_t* bm, int j) { return (bm[j >> 5] >> (j & 31)) & 1u; }

// Marks the top `r` tokens of [lo, hi) by `score` (skipping already marked
// tokens when `skip_marked`).
__device__ void select_tier(const float* score, int lo, int hi, int r, bool skip_marked, uint32_t* bm,
                            int* hist, int* wsum, int* shared2) {
  if (r <= 0) return;
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int above = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int d = tid; d < 256; d += kST) hist[d] = 0;
    __syncthreads();
    for (int j = lo + tid; j < hi; j += kST) {
      if (skip_marked && marked(bm, j)) continue;
      const uint32_t u = order_key(score[j]);
      if (pass > 0 && (u >> (shift + 8)) != (prefix >> (shift + 8))) continue;
      atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = above, digit = 0;
      for (int d = 255; d >= 0; --d) {
        if (cum + hist[d] >= r) {
          digit = d;
          break;
        }
        cum += hist[d];
      }
      shared2[0] = digit;
      shared2[1] = cum;
    }
    __syncthreads();
    prefix |= (uint32_t)shared2[0] << shift;
    above = shared2[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = r - above;  // >= 1 tokens equal to T, lowest indices first
  int taken_eq = 0;
  for (int base = lo; base < hi; base += kST) {
    const int j = base + tid;
    bool valid = j < hi;
    if (valid && skip_marked && marked(bm, j)) valid = false;
    const uint32_t u = valid ? order_key(score[j]) : 0u;
    const bool gt = valid && u > T;
    const bool eq = valid && u == T;
    int tot;
    const int before = block_prefix_count(eq, wsum, &tot);
    const bool take = gt || (eq && taken_eq + before < need_eq);
    if (take) atomicOr(&bm[j >> 5], 1u << (j & 31));
    taken_eq += tot;
    if (taken_eq >= need_eq && base + kST < hi) {
      // Remaining equal keys are not taken; only larger keys still are.
      for (int j2 = base + kST + tid; j2 < hi; j2 += kST) {
        if (skip_marked && marked(bm, j2)) continue;
        if (order_key(score[j2]) > T) atomicOr(&bm[j2 >> 5], 1u << (j2 & 31));
      }
      break;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kST) void select_kernel(SelParams p) {
  extern __shared__ uint32_t bm[];
  __shared__ int hist[256];
  __shared__ int wsum[kSWaves];
  __shared__ int shared2[2];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* ds = p.ds + (int64_t)b * p.ld;
  const float* ts = p.ts + (int64_t)b * p.ld;
  int32_t* out = p.out + (int64_t)b * p.k_out;
  const int L = p.L;
  if (p.budget >= L) {
    for (int j = tid; j < L; j += kST) out[j] = j;
    return;
  }
  const int lo = p.sink < L ? p.sink : L;
  const int w = p.window < L ? p.window : L;
  const int hi = L - w > lo ? L - w : lo;
  const int n_prot = lo + (L - hi);
  const int rest = p.budget - n_prot;
  const int n_free = hi - lo;
  int r1 = p.top_m < rest ? p.top_m : rest;
  r1 = r1 < n_free ? r1 : n_free;
  const int r2 = rest - r1;

  const int words = (L + 31) >> 5;
  for (int i = tid; i < words; i += kST) bm[i] = 0u;
  __syncthreads();
  select_tier(ds, lo, hi, r1, false, bm, hist, wsum, shared2);
  select_tier(ts, lo, hi, r2, true, bm, hist, wsum, shared2);

  int written = 0;
  for (int base = 0; base < L; base += kST) {
    const int j = base + tid;
    const bool sel = j < L && (j < lo || j >= hi || marked(bm, j));
    int tot;
    const int before = block_prefix_count(sel, wsum, &tot);
    if (sel && written + before < p.k_out) out[written + before] = j;
    written += tot;
  }
}

}  // namespace

size_t select_ws_bytes(int32_t, int32_t) { return 0; }

hipError_t launch_select(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                         int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                         void*, hipStream_t stream) {
  SelParams p{};
  p.ds = draft_score;
  p.ts = target_score;
  p.out = verify_idx;
  p.ld = ld;
  p.L = L;
  p.sink = sink;
  p.window = window;
  p.top_m = top_m;
  p.budget = budget;
  p.k_out = budget < L ? budget : L;
  const size_t lds = budget < L ? (size_t)((L + 31) / 32) * 4 : 4;
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3(B), dim3(kST), lds, stream, p);
  return hipGetLastError();
}

}  // namespace va
