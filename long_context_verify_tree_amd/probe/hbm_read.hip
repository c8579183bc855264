// Read-only HBM streaming probe (measurement only, not part of the
// verification path).  It gives the achievable read bandwidth of the device
// that the attention kernels' HBM fractions are compared with beside the
// vendor peak.  Built into its own library, libva_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte chunks with eight independent loads in
// flight per thread.  The XOR of everything read is stored only if it equals
// a fixed constant, which keeps the loads live without writing per thread.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Gathered-row read: for every (sequence, head) slab of `heads` per
// sequence, the rows idx[b, 0..K) of a K and a V array laid out
// [B, heads, L, row_bytes] (16 lanes per 256-byte row, eight chunks in
// flight per thread).  The same access pattern as a sparse verification's
// context reads, with no compute: the achievable rate for scattered rows.
// Indices outside [0, L) are not read.
__global__ __launch_bounds__(256) void gather_read_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                          const int32_t* __restrict__ idx, int heads, int K,
                                                          int L, int cpr, size_t n_items,
                                                          uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < n_items; i0 += U * stride) {
    u32x4 a[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = u32x4{0, 0, 0, 0};
      c[u] = u32x4{0, 0, 0, 0};
      const size_t it = i0 + u * stride;
      if (it < n_items) {
        const size_t row = it / cpr;               // (b, h, j)
        const int chunk = (int)(it % cpr);
        const int j = (int)(row % K);
        const size_t bh = row / K;
        const int b = (int)(bh / heads);
        const int ix = idx[(size_t)b * K + j];
        if ((unsigned)ix < (unsigned)L) {
          const size_t off = (bh * L + ix) * cpr + chunk;
          a[u] = __builtin_nontemporal_load(k + off);
          c[u] = __builtin_nontemporal_load(v + off);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w ^ c[u].x ^ c[u].y ^ c[u].z ^ c[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// Enqueue one gathered read: rows idx[b, 0..K) (int32, contiguous [B, K])
// of the [B, heads, L, row_bytes] device arrays k and v.  row_bytes is a
// multiple of 16.  Returns a hipError_t.
extern "C" int va_probe_gather_read(const void* k, const void* v, const int32_t* idx, int B, int heads, int K, int L,
                                    int row_bytes, uint32_t* sink, int grid, hipStream_t stream) {
  if (!k || !v || !idx || !sink || B <= 0 || heads <= 0 || K <= 0 || L <= 0 || row_bytes <= 0 || row_bytes % 16 ||
      grid <= 0)
    return (int)hipErrorInvalidValue;
  const int cpr = row_bytes / 16;
  const size_t n_items = (size_t)B * heads * K * cpr;
  hipLaunchKernelGGL(gather_read_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)k, (const u32x4*)v, idx,
                     heads, K, L, cpr, n_items, sink);
  return (int)hipGetLastError();
}

// Enqueue one read of `bytes` (a multiple of 16) from device memory `src` on
// `stream`; `sink` is 4 bytes of device memory.  Returns a hipError_t.
extern "C" int va_probe_hbm_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  if (!src || !sink || bytes % 16 || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(256), 0, stream, (const u32x4*)src, bytes / 16, sink);
  return (int)hipGetLastError();
}
