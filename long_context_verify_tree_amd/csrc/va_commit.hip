// Accept-and-commit (Dustin, "Workflow di Verifica" step 5): the accepted
// draft tokens are appended to the KV cache, the rejected ones dropped.
//
// The accepted tokens of a sequence are one root-to-node path of the draft
// tree; the kernel copies their K/V rows, root first, to positions
// cache_len[b], cache_len[b] + 1, ... of every KV head.  One workgroup per
// (sequence, KV head): the parent row is read into LDS, thread 0 walks the
// chain there, then the workgroup copies 16-byte chunks.  HBM-bound on a few rows per sequence,
// so in practice launch-latency bound.

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kCommitThreads = 256;
constexpr int kCommitMaxN = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams p) {
  __shared__ int path[kCommitMaxN];
  __shared__ int par[kCommitMaxN];
  __shared__ int plen;
  const int kvh = blockIdx.x % p.Hkv;
  const int b = blockIdx.x / p.Hkv;
  // the parent row in one coalesced read, then the walk in LDS
  for (int j = threadIdx.x; j < p.N; j += kCommitThreads) par[j] = p.parent[(int64_t)b * p.N + j];
  // The sequence's length is read before any store of this launch (the host
  // rejects an output length array that overlaps an input).
  const int base = p.cache_len[b];
  __syncthreads();
  if (threadIdx.x == 0) {
    const int leaf = p.accepted[b];
    int n = 0;
    if (leaf >= 0 && leaf < p.N) {
      // leaf first, then its ancestors; a malformed parent ends the path
      for (int j = leaf; j >= 0 && n < p.N;) {
        path[n++] = j;
        const int pj = par[j];
        j = (pj >= -1 && pj < j) ? pj : -1;
      }
      for (int i = 0; i < n / 2; ++i) {
        const int t = path[i];
        path[i] = path[n - 1 - i];
        path[n - 1 - i] = t;
      }
    }
    plen = n;
    if (kvh == 0) p.new_len[b] = base + n;
  }
  __syncthreads();
  const int n = plen;
  const int chunks = p.row_bytes / 16;
  unsigned char* kc = (unsigned char*)p.kc;
  unsigned char* vc = (unsigned char*)p.vc;
  const unsigned char* kd = (const unsigned char*)p.kd;
  const unsigned char* vd = (const unsigned char*)p.vd;
  for (int idx = threadIdx.x; idx < n * chunks; idx += kCommitThreads) {
    const int d = idx / chunks, c = idx % chunks;
    const int64_t pos = (int64_t)base + d;
    if (pos < 0 || pos >= p.capacity) continue;   // no room: the row is dropped
    const int node = path[d];
    const int64_t off = (int64_t)c * 16;
    const int64_t dk = ((int64_t)b * p.kcs[0] + (int64_t)kvh * p.kcs[1] + pos * p.kcs[2]) * p.es + off;
    const int64_t dv = ((int64_t)b * p.vcs[0] + (int64_t)kvh * p.vcs[1] + pos * p.vcs[2]) * p.es + off;
    const int64_t sk = ((int64_t)b * p.kds[0] + (int64_t)kvh * p.kds[1] + (int64_t)node * p.kds[2]) * p.es + off;
    const int64_t sv = ((int64_t)b * p.vds[0] + (int64_t)kvh * p.vds[1] + (int64_t)node * p.vds[2]) * p.es + off;
    *(u32x4*)(kc + dk) = *(const u32x4*)(kd + sk);
    *(u32x4*)(vc + dv) = *(const u32x4*)(vd + sv);
  }
}

}  // namespace

hipError_t launch_commit(const CommitParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3(p.B * p.Hkv), dim3(kCommitThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
