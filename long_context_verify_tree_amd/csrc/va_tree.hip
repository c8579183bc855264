// Best-first draft tree (BASTION, "Drafting a Diffusione a Blocchi Basato su
// Albero" and "Surrogato di Accettazione ed Espansione Best-First"): a block
// drafter gives, for each of K positions, T candidate tokens with marginal
// probabilities q_k; a node at depth d picks one candidate at each of the
// first d positions and scores rho = q_0 * ... * q_{d-1}.  The tree grows by
// adding, N times, the valid node of highest rho; adding a node makes its
// best child and its next sibling valid.  With marginals in [0, 1] rho
// never grows along a path, and the result is the N prefixes of largest
// rho, prefix-closed (the expansion below follows the rule for any input).
//
// One workgroup per sequence: the candidates are ranked per position in LDS
// (rank = number of better candidates, ties to the lower index), then one
// wavefront runs the expansion with the frontier in its registers, taking
// each step's best entry with DPP wavefront maxima over 64-bit keys (rho
// bits, then the earlier parent, then the better rank).

#include <stdint.h>

#include <type_traits>

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

// f(integral_constant<int, P>) for P = P0 .. S - 1, each a separate instance
template <int P0, int S, class F>
__device__ inline __attribute__((always_inline)) void for_phases(F& f) {
  if constexpr (P0 < S) {
    f(std::integral_constant<int, P0>{});
    for_phases<P0 + 1, S>(f);
  }
}

__device__ inline uint64_t entry_key(float rho, int par, int rank) {
  return ((uint64_t)__float_as_uint(rho) << 32) | ((uint64_t)(0xFFFFu - (uint32_t)(par + 1)) << 16) |
         (uint64_t)(0xFFFFu - (uint32_t)rank);
}

__global__ __launch_bounds__(kTreeThreads) void tree_kernel(TreeParams p) {
  __shared__ float praw[kTreeMaxKT];
  __shared__ float q[kTreeMaxKT];        // [k][rank], descending per position
  __shared__ int qt[kTreeMaxKT];
  __shared__ int opar[kTreeMaxN], otix[kTreeMaxN];   // parent; candidate (position * T + rank)
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

  // Expansion by wavefront 0.  The frontier holds, for each stream (the
  // root's candidates and then each added node's), its next candidate not
  // yet taken: node n's children are stream n + 1, taken in rank order, so
  // a step advances the winner's stream to its next rank (the "next
  // sibling") and opens the new node's stream at rank 0 (its "best child").
  // Stream s lives in lane s % 64, slot s / 64, with its head's 64-bit key
  // and its parent's rho, depth and rank; every lane keeps its best head.
  // The loop is unrolled over the slot that new streams open in, so every
  // register index is a compile-time constant and each update is a select.
  if (tid < 64) {
    const int lane = tid;
    constexpr int S = (kTreeMaxN + 1 + 63) / 64;   // slots per lane (streams <= N + 1)
    uint32_t khi[S], klo[S];   // head key (0: no candidate left)
    float srho[S];             // rho of the stream's parent (1 for the root)
    int sdep[S], srank[S];     // the parent's depth (candidates at that position); head rank
#pragma unroll
    for (int t = 0; t < S; ++t) {
      khi[t] = klo[t] = 0u;
      srho[t] = 0.f;
      sdep[t] = srank[t] = 0;
    }
    if (lane == 0) {   // stream 0: the root's candidates, best first
      const uint64_t k0 = entry_key(q[0], -1, 0);
      khi[0] = (uint32_t)(k0 >> 32);
      klo[0] = (uint32_t)k0;
      srho[0] = 1.f;
    }
    // this lane's best head over slots 0..last
    uint32_t bh = 0u, bl = 0u;
    int bsid = 0, bdep = 0, brank = 0;
    float brho = 0.f;
    auto rescan = [&](auto last_tag) __attribute__((always_inline)) {
      constexpr int LAST = decltype(last_tag)::value;
      bh = bl = 0u;
#pragma unroll
      for (int t = 0; t <= LAST; ++t) {
        const bool better = khi[t] > bh || (khi[t] == bh && klo[t] > bl);
        bh = better ? khi[t] : bh;
        bl = better ? klo[t] : bl;
        bsid = better ? 64 * t + lane : bsid;
        bdep = better ? sdep[t] : bdep;
        brank = better ? srank[t] : brank;
        brho = better ? srho[t] : brho;
      }
    };
    rescan(std::integral_constant<int, 0>{});
    int n = 0;
    auto phase = [&](auto phase_tag) __attribute__((always_inline)) {
      constexpr int P = decltype(phase_tag)::value;
      // phase P: the new node's stream n + 1 opens in slot P
      while (n < N && ((n + 1) >> 6) == P) {
        // the winner: largest rho bits, then the largest tie bits among
        // those (keys are unique), then the lane that holds it
        const uint32_t hi = wave_max_u32(bh);
        const uint64_t cand = __ballot(bh == hi);
        int owner;
        if (__builtin_popcountll(cand) > 1) {
          const uint32_t lo = wave_max_u32(bh == hi ? bl : 0u);
          owner = (int)__builtin_ctzll(__ballot(bh == hi && bl == lo));
        } else {
          owner = (int)__builtin_ctzll(cand);
        }
        const int w = __builtin_amdgcn_readlane(bsid, owner);      // winning stream
        const int dp = __builtin_amdgcn_readlane(bdep, owner);     // its parent's depth
        const int r = __builtin_amdgcn_readlane(brank, owner);     // the candidate's rank
        const float rp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(brho), owner));
        const float rho_n = __uint_as_float(hi);                   // rp * q[dp][r], as keyed
        const bool adv = r + 1 < T, child = dp + 1 < K;
        const float qa = adv ? q[dp * T + r + 1] : 0.f;
        const float qc = child ? q[(dp + 1) * T] : 0.f;
        if (lane == 0) {
          opar[n] = w - 1;
          orho[n] = rho_n;
          otix[n] = dp * T + r;
        }
        // the winner's stream moves to its next rank
        const uint64_t ka = adv ? entry_key(rp * qa, w - 1, r + 1) : 0ull;
        const bool mine = lane == (w & 63);
#pragma unroll
        for (int t = 0; t <= P; ++t) {
          const bool sel = mine && t == (w >> 6);
          khi[t] = sel ? (uint32_t)(ka >> 32) : khi[t];
          klo[t] = sel ? (uint32_t)ka : klo[t];
          srank[t] = sel ? r + 1 : srank[t];
        }
        // the new node's stream opens at its best child
        const uint64_t kc = child ? entry_key(rho_n * qc, n, 0) : 0ull;
        const bool opens = lane == ((n + 1) & 63);
        khi[P] = opens ? (uint32_t)(kc >> 32) : khi[P];
        klo[P] = opens ? (uint32_t)kc : klo[P];
        srho[P] = opens ? rho_n : srho[P];
        sdep[P] = opens ? dp + 1 : sdep[P];
        srank[P] = opens ? 0 : srank[P];
        rescan(std::integral_constant<int, P>{});
        ++n;
      }
    };
    for_phases<0, S>(phase);
    if (lane == 0) {
      float a = 0.f;
      for (int m = 0; m < N; ++m) a += orho[m];
      p.a_hat[b] = a;
    }
  }
  __syncthreads();
  for (int m = tid; m < N; m += kTreeThreads) {
    p.parent[(int64_t)b * N + m] = opar[m];
    p.token[(int64_t)b * N + m] = qt[otix[m]];
    p.rho[(int64_t)b * N + m] = orho[m];
  }
}

}  // namespace

hipError_t launch_tree(const TreeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(tree_kernel, dim3(p.B), dim3(kTreeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace va
