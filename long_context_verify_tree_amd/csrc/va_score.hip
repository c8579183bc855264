// Importance scores for the verify-set selector (Dustin, "Metodologia"
// sections 1-2): attention scores of a few scoring heads, aggregated into one
// global importance map per sequence,
//
//     score[b, j] = sum_{h < Hs} sum_{i < M} softmax_j(scale * <q[b,h,i], k[b,h,j]>),
//
// the softmax taken over the L context tokens.  A row's softmax needs its
// log-sum-exp over all of L before any probability is final, so the work is
// two kernels:
//   score_partial_kernel  one workgroup per (sequence, head, split of L);
//                         each wavefront keeps two K tiles in flight in
//                         registers; S^T = K_tile . Q^T on MFMA for up to
//                         32 rows,
//                         writes the scaled scores (log2 domain) to the
//                         workspace and each row's (max, sum) of the split;
//   score_finish_kernel   one workgroup per (sequence, 1024 tokens): merges
//                         the split statistics into each row's log2-sum-exp,
//                         then sums exp2(S - lse) over the rows per token.
// K is read once (HBM-bound); keeping S costs 4·M bytes per token and head
// against 2·D bytes of K, and saves a second pass over K.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "va_device.h"
#include "va_internal.h"

namespace va {
namespace {

using namespace dev;

constexpr int kSWavesS = 4;
constexpr int kSThreads = 64 * kSWavesS;
constexpr int kSTile = 32;     // keys per tile
constexpr int kFinishTokens = 1024;

template <int D>
__global__ __launch_bounds__(kSThreads) void score_partial_kernel(ScoreParams p) {
  constexpr int VEC = 8;
  constexpr int CPR = D / VEC;
  constexpr int NCH = kSTile * CPR / 64;   // 16-byte chunks per lane per tile
  constexpr int KPC = 64 / CPR;            // key rows between a lane's chunks
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kSWavesS][kSTile * D];
  __shared__ float mbuf[kSWavesS][32], lbuf[kSWavesS][32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n = lane & 31;
  int id = xcd_remap(blockIdx.x, p.total_groups);
  const int split = id % p.n_splits;
  id /= p.n_splits;
  const int hs = id % p.Hs;
  const int b = id / p.Hs;
  const int kb = split * p.split_len;
  const int ke = min(p.L, kb + p.split_len);
  const int ntiles = ke > kb ? (ke - kb + kSTile - 1) / kSTile : 0;

  // queries of the up to 32 rows as MFMA B operands (rows >= M are zero)
  bf16x8 qop[KS];
  {
    const bool ok = n < p.M;
    const uint16_t* qrow = (const uint16_t*)p.q + (int64_t)b * p.qs[0] + (int64_t)hs * p.qs[1] + (int64_t)(ok ? n : 0) * p.qs[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = ok ? *(const u32x4*)(qrow + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)b * p.ks[0] + (int64_t)hs * p.ks[1];
  const uint32_t kts_b = (uint32_t)(p.ks[2] * 2);
  const rsrc_t krs = make_rsrc(kbase, (uint32_t)p.L * kts_b);
  const int kk0 = lane / CPR;
  const uint32_t col_b = (uint32_t)(lane % CPR) * 16u;
  uint16_t* kt = tiles[wave];
  float* srow = p.s + ((int64_t)(b * p.Hs + hs) * p.M + n) * p.ld_s;

  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;
  // Wave w takes tiles w, w + 4, ...: its i-th tile is w + 4 i.  A ring of
  // two register tiles keeps the next two in flight while one is used;
  // slots past the part's last tile load nothing (out-of-range offset).
  constexpr int RING = 2;
  const int nt_w = ntiles > wave ? (ntiles - wave + kSWavesS - 1) / kSWavesS : 0;
  u32x4 kr[RING][NCH];
  auto load = [&](u32x4 (&rx)[NCH], int i) __attribute__((always_inline)) {
    const int t = wave + kSWavesS * i;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const uint32_t off = (uint32_t)(kb + kSTile * t + kk0 + KPC * cc) * kts_b + col_b;
      rx[cc] = buf_load16<true>(krs, i < nt_w ? off : kOOB);   // past L: zeros
    }
  };
  auto process = [&](u32x4 (&rx)[NCH], int i) __attribute__((always_inline)) {
    const int t = wave + kSWavesS * i;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int kk = kk0 + KPC * cc;
      *(u32x4*)(kt + kk * D + swz<CPR>(kk, lane % CPR) * VEC) = rx[cc];
    }
    load(rx, i + RING);   // refill the slot while this tile is used
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kv = *(const u32x4*)(kt + n * D + swz<CPR>(n, 2 * ks + h) * VEC);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qop[ks], s, 0, 0, 0);
    }
    // lane (n, h) holds row n's keys 8g + 4h + r (e = 4g + r) of the tile
    const int key0 = kb + kSTile * t;
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + 8 * (e >> 2) + 4 * h + (e & 3);
      s[e] = key < ke ? s[e] * c : -INFINITY;
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = half_max(tmax);
    const float mnew = fmaxf(m_run, tmax);
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ls += fast_exp2(s[e] - mnew);
    ls = half_sum(ls);
    l_run = (m_run == -INFINITY ? 0.f : l_run * fast_exp2(m_run - mnew)) + ls;
    m_run = mnew;
    if (n < p.M) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(srow + key0 + 8 * g + 4 * h) = make_float4(s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]);
    }
  };
#pragma unroll
  for (int r = 0; r < RING; ++r) load(kr[r], r);
  // whole turns of the ring (no early exit inside), then the odd last tile
  int i = 0;
  for (; i + RING <= nt_w; i += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) process(kr[r], i + r);
  }
  if (i < nt_w) process(kr[0], i);
  // the four wavefronts' (max, sum) of each row, in a fixed order
  if (h == 0) {
    mbuf[wave][n] = m_run;
    lbuf[wave][n] = l_run;
  }
  __syncthreads();
  if (tid < 32 && tid < p.M) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSWavesS; ++w) M = fmaxf(M, mbuf[w][tid]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kSWavesS; ++w)
      l += mbuf[w][tid] == -INFINITY ? 0.f : lbuf[w][tid] * fast_exp2(mbuf[w][tid] - M);
    const int64_t r = (int64_t)(b * p.Hs + hs) * p.M + tid;
    p.stat_m[r * p.n_splits + split] = M;
    p.stat_l[r * p.n_splits + split] = l;
  }
}

__global__ __launch_bounds__(256) void score_finish_kernel(ScoreParams p) {
  extern __shared__ float lse2[];   // [Hs * M]
  const int tid = threadIdx.x;
  const int chunks = (p.L + kFinishTokens - 1) / kFinishTokens;
  const int b = blockIdx.x / chunks;
  const int j0 = (blockIdx.x % chunks) * kFinishTokens;
  const int R = p.Hs * p.M;
  for (int r = tid; r < R; r += 256) {
    const int64_t row = (int64_t)b * R + r;
    float M = -INFINITY;
#pragma unroll 8
    for (int sp = 0; sp < p.n_splits; ++sp) M = fmaxf(M, p.stat_m[row * p.n_splits + sp]);
    float l = 0.f;
#pragma unroll 8
    for (int sp = 0; sp < p.n_splits; ++sp) {
      const float ms = p.stat_m[row * p.n_splits + sp];
      l += ms == -INFINITY ? 0.f : p.stat_l[row * p.n_splits + sp] * fast_exp2(ms - M);
    }
    lse2[r] = M + log2f(l);
  }
  __syncthreads();
  const int j = j0 + 4 * tid;
  if (j >= p.L) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const float* sb = p.s + (int64_t)b * R * p.ld_s + j;
  // unrolled so that eight rows' loads are in flight at once (the sum keeps
  // its row order)
#pragma unroll 8
  for (int r = 0; r < R; ++r) {
    const float4 v = *(const float4*)(sb + (int64_t)r * p.ld_s);   // rows padded to 32 tokens
    const float z = lse2[r];
    acc[0] += fast_exp2(v.x - z);
    acc[1] += fast_exp2(v.y - z);
    acc[2] += fast_exp2(v.z - z);
    acc[3] += fast_exp2(v.w - z);
  }
  float* out = p.score + (int64_t)b * p.ld_out;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (j + e < p.L) out[j + e] = acc[e];
}

// Attention Recovery Rate of a verify set (Dustin, "Metodologia" section
// 2): the share of the importance map of all verification rows that falls
// on the set, arr[b] (+)= sum_k score[b, idx[b, k]] / rows.  One workgroup per
// sequence; each thread sums a fixed strided subset of the set, then a fixed
// reduction tree (bitwise reproducible).  Indices outside [0, L) add 0.
__global__ __launch_bounds__(256) void recovery_kernel(const float* score, int64_t ld, int L, const int32_t* idx,
                                                       int K, int64_t idx_stride, float inv_rows, int accumulate,
                                                       float* arr) {
  __shared__ float part[256];
  const int b = blockIdx.x;
  const float* srow = score + (int64_t)b * ld;
  const int32_t* irow = idx + (int64_t)b * idx_stride;
  float acc = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) {
    const int j = irow[k];
    acc += (unsigned)j < (unsigned)L ? srow[j] : 0.f;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) arr[b] = (accumulate ? arr[b] : 0.f) + part[0] * inv_rows;
}

}  // namespace

hipError_t launch_recovery(const float* score, int64_t ld, int B, int L, const int32_t* idx, int K,
                           int64_t idx_stride, int rows, int accumulate, float* arr, hipStream_t stream) {
  hipLaunchKernelGGL(recovery_kernel, dim3(B), dim3(256), 0, stream, score, ld, L, idx, K, idx_stride,
                     1.0f / (float)rows, accumulate, arr);
  return hipGetLastError();
}

hipError_t launch_scores(const ScoreParams& p, int D, hipStream_t stream) {
  if (D == 64)
    hipLaunchKernelGGL(score_partial_kernel<64>, dim3(p.total_groups), dim3(kSThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(score_partial_kernel<128>, dim3(p.total_groups), dim3(kSThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunks = (p.L + kFinishTokens - 1) / kFinishTokens;
  hipLaunchKernelGGL(score_finish_kernel, dim3(p.B * chunks), dim3(256), (size_t)p.Hs * p.M * sizeof(float), stream,
                     p);
  return hipGetLastError();
}

}  // namespace va
