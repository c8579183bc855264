// Device helpers shared by the HIP kernels of libverify_attn.so: vector
// types, XCD-aware workgroup ids, the LDS-only barrier, the LDS chunk
// swizzle and raw-buffer K/V reads.  Internal; included by the .hip files
// inside namespace va.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace va {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte vector used for every global/LDS move.  may_alias: LDS tiles are
// written through this type and read back as bf16 / float elements.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), __may_alias__));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), __may_alias__));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ inline int xcd_remap(int x, int total) {
  // Workgroups are dispatched round-robin over the 8 XCDs (x % 8).  Give each
  // XCD a contiguous range of logical ids so neighbours (row tiles of one
  // split) share that XCD's L2.
  const int q = total / 8, r = total % 8;
  const int xcd = x % 8, local = x / 8;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum and sum of x over lanes l and l ^ 32, through the cross-half lane
// swap (a VALU operation, no LDS round trip).  Of the swap's two results, in
// every lane one holds x of lanes 0-31 and the other x of lanes 32-63, so
// both halves combine the same two values in the same order.
__device__ inline void half_swap(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  lo = __builtin_bit_cast(float, (uint32_t)r[0]);
  hi = __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ inline float half_max(float x) {
  float lo, hi;
  half_swap(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ inline float half_sum(float x) {
  float lo, hi;
  half_swap(x, lo, hi);
  return lo + hi;
}

// Workgroup barrier for LDS hand-offs inside the streaming loops.
// __syncthreads() is a workgroup release/acquire fence and waits for every
// outstanding global load too, which would drain the register prefetch ring
// at each tile; this waits only for this wavefront's LDS operations
// (lgkmcnt(0)) before the hardware barrier.  The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Bank-conflict swizzle of the 16-byte chunks of a key row in LDS.
template <int CPR>
__device__ inline int swz(int row, int chunk) {
  return chunk ^ (row & (CPR - 1));
}

// Buffer resources for K/V reads.  A raw buffer load whose byte offset is
// at or past the resource's size returns zeros without touching memory, so
// keys past the end of a part (and gathered indices outside [0, L), given
// the offset kOOB) need neither clamps nor zero fills, and every load takes
// one 32-bit offset instead of a 64-bit address.  The host keeps each K/V
// region of one (sequence, kv head) under 2^31 bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;
// The base and size are wavefront-uniform; readfirstlane states it, so the
// resource lives in scalar registers (a per-lane resource would make the
// compiler wrap every load in a loop over distinct values).
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// buf_load16<true> carries the non-temporal hint (cache-policy bit `nt`)
// for K/V rows that are read exactly once per call: they then do not
// displace the workspace and query lines in L2 (partial kernel on the
// Llama-3-8B 32k workload: 193 -> 178 us).  Rows that another row tile reads
// again take the default policy: there the second read is an L2 hit.
template <bool NT = false>
__device__ inline u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, NT ? 2 : 0));
}
__device__ inline int buf_load_i32(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

}  // namespace dev
}  // namespace va
