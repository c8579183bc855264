// Best-first draft tree (BASTION, "Drafting a Diffusione a Blocchi Basato su
// Albero" and "Surrogato di Accettazione ed Espansione Best-First"): a block
// drafter gives, for each of K positions, T candidate tokens with marginal
// probabilities q_k; a node at depth d picks one candidate at each of the
// first d positions and scores rho = q_0 * ... * q_{d-1}.  The tree grows by
// adding, N times, the valid node of highest rho; adding a node makes its
// best child and its next sibling valid.  Since rho never grows along a
// path, the result is the N prefixes of largest rho, prefix-closed.
//
// One workgroup per sequence: the candidates are ranked per position in LDS
// (rank = number of better candidates, ties to the lower index), then one
// wavefront runs the expansion over an LDS frontier (at most 2N + 1
// entries), taking each step's best entry with DPP wavefront maxima over
// 64-bit keys (rho bits, then the earlier parent, then the better rank).

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "va_internal.h"

namespace va {
namespace {

constexpr int kTreeThreads = 256;

__device__ inline float sane(float x) { return x > 0.f ? x : 0.f; }   // NaN and negatives count as 0

// Maximum of v over the wavefront, returned to every lane: DPP prefix max
// within each 16-lane row (shifts 1, 2, 4, 8), then across rows with the
// row broadcasts; lane 63 ends with the total.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline uint64_t entry_key(float rho, int par, int rank) {
  return ((uint64_t)__float_as_uint(rho) << 32) | ((uint64_t)(0xFFFFu - (uint32_t)(par + 1)) << 16) |
         (uint64_t)(0xFFFFu - (uint32_t)rank);
}

__global__ __launch_bounds__(kTreeThreads) void tree_kernel(TreeParams p) {
  __shared__ float praw[kTreeMaxKT];
  __shared__ float q[kTreeMaxKT];        // [k][rank], descending per position
  __shared__ int qt[kTreeMaxKT];
  __shared__ uint64_t fkey[2 * kTreeMaxN + 1];
  __shared__ int fpar[2 * kTreeMaxN + 1], frank[2 * kTreeMaxN + 1], fdepth[2 * kTreeMaxN + 1];
  __shared__ float frho[2 * kTreeMaxN + 1];   // rho of the entry's parent (1 for the root)
  __shared__ int opar[kTreeMaxN], otok[kTreeMaxN];
  __shared__ float orho[kTreeMaxN];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int K = p.K, T = p.T, N = p.N, KT = p.K * p.T;
  const float* prob = p.prob + (int64_t)b * KT;
  const int32_t* tok = p.tok + (int64_t)b * KT;

  for (int e = tid; e < KT; e += kTreeThreads) praw[e] = sane(prob[e]);
  __syncthreads();
  for (int e = tid; e < KT; e += kTreeThreads) {
    const int k = e / T, j = e % T;
    const float pj = praw[e];
    int r = 0;
    for (int j2 = 0; j2 < T; ++j2) {
      const float p2 = praw[k * T + j2];
      r += (p2 > pj) || (p2 == pj && j2 < j);
    }
    q[k * T + r] = pj;
    qt[k * T + r] = tok[e];
  }
  __syncthreads();

  if (tid < 64) {
    const int lane = tid;
    int nf = 1;
    if (lane == 0) {
      fkey[0] = entry_key(q[0], -1, 0);
      fpar[0] = -1;
      frank[0] = 0;
      fdepth[0] = 1;
      frho[0] = 1.f;
    }
    __builtin_amdgcn_wave_barrier();
    for (int n = 0; n < N; ++n) {
      uint64_t best = 0;
      int bi = 0;
      for (int i = lane; i < nf; i += 64) {
        const uint64_t k = fkey[i];
        if (k > best) {
          best = k;
          bi = i;
        }
      }
      // the winner: largest rho bits, then the largest tie bits among those
      // (keys are unique), then the lane that holds it
      const uint32_t hi = wave_max_u32((uint32_t)(best >> 32));
      const uint32_t lo = wave_max_u32((uint32_t)(best >> 32) == hi ? (uint32_t)best : 0u);
      const uint64_t owner = __ballot((uint32_t)(best >> 32) == hi && (uint32_t)best == lo);
      bi = __builtin_amdgcn_readlane(bi, (int)__builtin_ctzll(owner));
      // every lane holds the same winner; read it and take the same steps
      const int par = fpar[bi], rank = frank[bi], depth = fdepth[bi];
      const float rho_par = frho[bi];
      const float r = rho_par * q[(depth - 1) * T + rank];
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        opar[n] = par;
        otok[n] = qt[(depth - 1) * T + rank];
        orho[n] = r;
        fkey[bi] = 0;
      }
      if (depth < K) {   // best child
        if (lane == 0) {
          fkey[nf] = entry_key(r * q[depth * T], n, 0);
          fpar[nf] = n;
          frank[nf] = 0;
          fdepth[nf] = depth + 1;
          frho[nf] = r;
        }
        ++nf;
      }
      if (rank + 1 < T) {   // next sibling
        if (lane == 0) {
          fkey[nf] = entry_key(rho_par * q[(depth - 1) * T + rank + 1], par, rank + 1);
          fpar[nf] = par;
          frank[nf] = rank + 1;
          fdepth[nf] = depth;
          frho[nf] = rho_par;
        }
        ++nf;
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) {
      float a = 0.f;
      for (int n = 0; n < N; ++n) a += orho[n];
      p.a_hat[b] = a;
    }
  }
  __syncthreads();
  for (int n = tid; n < N; n += kTreeThreads) {
    p.parent[(int64_t)b * N + n] = opar[n];
    p.token[(int64_t)b * N + n] = otok[n];
    p.rho[(int64_t)b * N + n] = orho[n];
  }
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(tree_kernel, dim3(p.B), dim3(kTreeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
