// Verify-set selection for sparse verification (Dustin, "Aggregazione
// Ibrida dell'Attenzione"): keep the attention-sink prefix and the local
// window, take the top-m tokens by draft-lookahead score, then fill the rest
// of the budget with the best remaining tokens by target-historical score.
//
// One workgroup of 1024 threads per sequence.  The row is cut into segments
// of 32768 tokens; in each segment thread t owns the 32 consecutive tokens
// 32t .. 32t+31, so "lower index first" is thread order and then bit order,
// and one 32-bit word per thread and segment holds the thread's selection
// marks.  Each tier is an exact top-r over the candidates (tokens between
// sink and window, minus those already taken):
//   * scores become order-preserving 32-bit keys (NaN lowest, -0 == +0);
//   * three radix passes (12, 10 and 10 bits) over LDS histograms (integer
//     atomics, so counts do not depend on thread order) find the key T of the
//     r-th best candidate and the number of candidates strictly above it.
//     The first pass of both tiers shares one sweep: the target histogram
//     counts every free token, and the draft tier's picks are subtracted
//     from it before the target tier starts;
//   * one block-wide exclusive scan of each thread's count of keys equal to
//     T gives every such token its rank in index order; the first ones up to
//     r are taken (the lower-index tie rule).
// A last block scan of the per-thread mark counts (plus sink and window)
// writes the ascending index list.  A row of one segment keeps its keys in
// registers for all passes; longer rows re-read each segment per pass (the
// row then sits in L2).  Rows longer than one segment go to a second kernel
// instead (select_cluster_kernel, below) when the batch is small enough:
// several workgroups per row, each holding 16384 tokens in registers.

#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "va_select.h"

namespace va {
namespace {

constexpr int kST = 1024;                 // threads per workgroup
constexpr int kSWaves = kST / 64;
constexpr int kKPT = 32;                  // tokens per thread per segment
constexpr int kSeg = kST * kKPT;          // tokens per segment
static_assert(kSeg == kSelectSegTokens, "segment size of the length limit");

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

// Exclusive prefix sum of v over the workgroup in thread order; *total gets
// the sum.  Uses wsum[kSWaves]; two barriers, or one with TAIL = false when
// the caller reaches another barrier before wsum is written again.
// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves (no
// LDS round trip): shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes
// without a source read 0), then lane 15 of rows 0 and 2 is added to rows 1
// and 3, and lane 31 to rows 2 and 3.
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

template <bool TAIL = true, int NW = kSWaves>
__device__ inline int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  if (TAIL) __syncthreads();
  *total = tot;
  return before + x - v;
}

// Radix digits of a 32-bit key: 12 bits, then 10, then 10.
constexpr int kDigitBits[3] = {12, 10, 10};
constexpr int kDigitShift[3] = {20, 10, 0};
constexpr int kBins0 = 1 << 12;

struct SelShared {
  int hist_d[kBins0];        // first-digit histogram of the draft tier
  int hist_t[kBins0];        // first-digit histogram of the target tier
  int hist_p[2][2][1 << 10]; // [tier][pass - 1]: later digits, zeroed with the others at the start
  int wsum[kSWaves];
  int pick[2];               // digit, candidates in higher buckets
};

// Bits of the 32 tokens [j0, j0 + 32) that lie in [lo, hi).
__device__ inline uint32_t range_bits(int j0, int lo, int hi) {
  const int a = lo - j0, e = hi - j0;   // bit i set for a <= i < e
  const uint32_t below_e = e <= 0 ? 0u : (e >= 32 ? ~0u : (1u << e) - 1u);
  const uint32_t below_a = a <= 0 ? 0u : (a >= 32 ? ~0u : (1u << a) - 1u);
  return below_e & ~below_a;
}

// Given a histogram of `nbins` buckets (nbins / kST per thread, highest
// buckets at the lowest threads) and `above` candidates in higher buckets
// already, finds the bucket holding the r-th largest candidate: sets
// sh.pick = {bucket, candidates above it}.  Two barriers; every thread
// reads the result after the last, which also orders the next use of wsum.
__device__ inline void pick_bucket(const int* hist, int nbins, int r, int above, SelShared& sh) {
  const int tid = threadIdx.x;
  const int per = nbins / kST;   // 4 or 1
  const int top = nbins - per * tid;   // this thread's buckets: [top - per, top)
  int c[4] = {0, 0, 0, 0};
  int csum = 0;
  for (int k = 0; k < per; ++k) {
    c[k] = hist[top - 1 - k];
    csum += c[k];
  }
  int tot;
  int cum = above + block_excl_scan<false>(csum, sh.wsum, &tot);
  if (cum < r && cum + csum >= r) {
    int bucket = top - 1;
    for (int k = 0; k < per; ++k) {
      if (cum + c[k] >= r) {
        bucket = top - 1 - k;
        break;
      }
      cum += c[k];
    }
    sh.pick[0] = bucket;
    sh.pick[1] = cum;
  }
  __syncthreads();
}

static_assert(sizeof(SelShared) + (size_t)(kSelectMaxL / kSeg) * kST * sizeof(uint32_t) <= 160 * 1024,
              "histograms and the mark words of the longest row must fit in LDS");

template <bool RESIDENT>
__global__ __launch_bounds__(kST) void select_kernel(SelParams p) {
  extern __shared__ uint32_t marks[];   // [nseg][kST]: tokens taken by the two tiers
  __shared__ SelShared sh;
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
  const int nseg = RESIDENT ? 1 : (L + kSeg - 1) / kSeg;

  for (int s = 0; s < nseg; ++s) marks[s * kST + tid] = 0u;
  for (int i = tid; i < kBins0; i += kST) {
    sh.hist_d[i] = 0;
    sh.hist_t[i] = 0;
    (&sh.hist_p[0][0][0])[i] = 0;
  }

  uint32_t kd[kKPT], kt[kKPT];
  auto load_keys = [&](const float* row, int s, uint32_t (&key)[kKPT]) __attribute__((always_inline)) {
    const int j0 = s * kSeg + tid * kKPT;
    const bool vec = j0 + kKPT <= L && ((reinterpret_cast<uintptr_t>(row + j0) & 15u) == 0);
    if (vec) {
#pragma unroll
      for (int q = 0; q < kKPT / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(row + j0 + 4 * q);
        key[4 * q + 0] = order_key(v.x);
        key[4 * q + 1] = order_key(v.y);
        key[4 * q + 2] = order_key(v.z);
        key[4 * q + 3] = order_key(v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) key[i] = j0 + i < L ? order_key(row[j0 + i]) : 0u;
    }
  };
  auto free_bits = [&](int s) __attribute__((always_inline)) -> uint32_t {
    return range_bits(s * kSeg + tid * kKPT, lo, hi);
  };

  // first digit of both tiers in one sweep; the target histogram counts
  // every free token and is corrected for the draft tier's picks later
  if (RESIDENT) {
    load_keys(ds, 0, kd);
    load_keys(ts, 0, kt);
  }
  __syncthreads();
  for (int s = 0; s < nseg; ++s) {
    if (!RESIDENT) {
      load_keys(ds, s, kd);
      load_keys(ts, s, kt);
    }
    const uint32_t cand = free_bits(s);
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      if ((cand >> i) & 1u) {
        if (r1 > 0) atomicAdd(&sh.hist_d[kd[i] >> kDigitShift[0]], 1);
        if (r2 > 0) atomicAdd(&sh.hist_t[kt[i] >> kDigitShift[0]], 1);
      }
    }
  }
  __syncthreads();

  // Marks the top r candidates (free tokens not yet marked) of a tier whose
  // first-digit histogram is hist0; key holds the keys when resident.
  auto tier = [&](const float* row, int r, int* hist0, int (&histp)[2][1 << 10], uint32_t (&key)[kKPT])
                  __attribute__((always_inline)) {
    uint32_t prefix = 0;
    int above = 0;
    pick_bucket(hist0, kBins0, r, 0, sh);
    prefix = (uint32_t)sh.pick[0] << kDigitShift[0];
    above = sh.pick[1];
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = kDigitShift[pass];
      const int nb = 1 << kDigitBits[pass];
      const int hs = shift + kDigitBits[pass];   // bits above this digit are fixed
      int* hist = histp[pass - 1];               // zeroed at the start
      for (int s = 0; s < nseg; ++s) {
        if (!RESIDENT) load_keys(row, s, key);
        const uint32_t cand = free_bits(s) & ~marks[s * kST + tid];
#pragma unroll
        for (int i = 0; i < kKPT; ++i) {
          if (((cand >> i) & 1u) && (key[i] >> hs) == (prefix >> hs))
            atomicAdd(&hist[(key[i] >> shift) & (uint32_t)(nb - 1)], 1);
        }
      }
      __syncthreads();
      pick_bucket(hist, nb, r, above, sh);
      prefix |= (uint32_t)sh.pick[0] << shift;
      above = sh.pick[1];
    }
    // every candidate above T, and the first (r - above) equal to T in
    // index order
    const uint32_t T = prefix;
    const int need_eq = r - above;
    int seen_eq = 0;
    for (int s = 0; s < nseg; ++s) {
      if (!RESIDENT) load_keys(row, s, key);
      const uint32_t cand = free_bits(s) & ~marks[s * kST + tid];
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int i = 0; i < kKPT; ++i) {
        const bool c = (cand >> i) & 1u;
        gt |= (uint32_t)(c && key[i] > T) << i;
        eq |= (uint32_t)(c && key[i] == T) << i;
      }
      int tot;
      const int before = seen_eq + block_excl_scan(__popc(eq), sh.wsum, &tot);
      int take = need_eq - before;   // equal keys this thread may still take
      uint32_t eq_taken = 0;
      for (uint32_t e = eq; e && take > 0; e &= e - 1, --take) eq_taken |= e & (~e + 1u);
      marks[s * kST + tid] |= gt | eq_taken;
      seen_eq += tot;
    }
  };

  if (r1 > 0) tier(ds, r1, sh.hist_d, sh.hist_p[0], kd);
  if (r2 > 0) {
    if (r1 > 0) {
      // take the draft tier's picks out of the target histogram
      for (int s = 0; s < nseg; ++s) {
        if (!RESIDENT) load_keys(ts, s, kt);
        const uint32_t m = marks[s * kST + tid];
#pragma unroll
        for (int i = 0; i < kKPT; ++i)
          if ((m >> i) & 1u) atomicSub(&sh.hist_t[kt[i] >> kDigitShift[0]], 1);
      }
      __syncthreads();
    }
    tier(ts, r2, sh.hist_t, sh.hist_p[1], kt);
  }

  // ascending output: sink, both tiers and window
  int written = 0;
  for (int s = 0; s < nseg; ++s) {
    const int j0 = s * kSeg + tid * kKPT;
    const uint32_t valid = range_bits(j0, 0, L);
    const uint32_t sel = (marks[s * kST + tid] | (valid & ~range_bits(j0, lo, hi))) & valid;
    int tot;
    const int before = written + block_excl_scan(__popc(sel), sh.wsum, &tot);
    int pos = before;
    for (uint32_t e = sel; e; e &= e - 1) {
      const int i = __ffs(e) - 1;
      if (pos < p.k_out) out[pos] = j0 + i;
      ++pos;
    }
    written += tot;
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup selection.  A row of P >= 2 segments of kCSeg tokens is
// split over P workgroups of kCT threads, one per segment; each holds its
// segment's keys in registers (thread t: tokens 32t .. 32t+31 of the
// segment, as above) and runs the same steps as select_kernel.  The
// workgroups of a row meet at row barriers, where
//   * the histograms of each radix pass are summed in the row's workspace
//     (integer atomics of each workgroup's nonzero LDS bins), and every
//     workgroup reads the sums back and takes the same bucket;
//   * the counts of equal keys and of output tokens are published per
//     segment, so each workgroup knows how many precede it in index order.
// A row barrier is an arrival counter in the workspace: each workgroup adds
// one and waits until all P have arrived for this phase.  The waits rely on
// every workgroup of the launch being resident at once: the host takes this
// kernel only when the occupancy API says the device holds B * P of its
// workgroups at once (else one workgroup per row).  Work on other streams
// can still hold CUs, so each wait is bounded: a timeout sets the row's
// error flag and the wave moves on, so every wave exits; the last workgroup
// of the row to finish (a counter bumped once its output stores are
// performed) then overwrites the whole row with -1, which the caller sees in
// place of a verify set.

#ifndef VA_SEL_CT
#define VA_SEL_CT 512   // 128: 83 us, 256: 64 us, 512: 58 us, 1024: 69 us on 4 rows of 131072
#endif
constexpr int kCT = VA_SEL_CT;             // threads per workgroup
constexpr int kCWaves = kCT / 64;
constexpr int kCSeg = kCT * kKPT;          // 16384 tokens per workgroup
constexpr int kCMaxGroups = 256;           // B * P limit: every workgroup resident (one per CU; two fit)
constexpr int kSpinLimit = 1 << 18;        // polls per wait (each a device-coherent load: < 1 s)

// Workspace of one row, in ints, zeroed before the launch.
constexpr int kWsHd = 0;                   // first digit, draft tier [kBins0]
constexpr int kWsHt = kBins0;              // first digit, target tier [kBins0]
constexpr int kWsHp = 2 * kBins0;          // later digits [tier][pass - 1][1024]
constexpr int kWsBar = kWsHp + 4 * 1024;   // arrival counter
constexpr int kWsErr = kWsBar + 1;         // set when a wait timed out
constexpr int kWsDone = kWsBar + 2;        // workgroups whose output stores are performed
constexpr int kWsCnt = kWsBar + 64;        // per segment: equal keys [2][P], output tokens [P]

__host__ __device__ inline int64_t cluster_row_ints(int P) { return ((int64_t)kWsCnt + 3 * P + 63) / 64 * 64; }

struct CShared {
  int ha[kBins0];     // a workgroup histogram, then the row's sums for a pick
  int hb[kBins0];
  int wsum[kCWaves];
  int pick[2];
};

__device__ inline int ld_dev(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// Returns once every workgroup of the row has reached its `phase`-th
// barrier (or the wait timed out).  Everything the workgroups exchange is
// written with agent-scope atomics (performed where every XCD sees them) and
// read with agent-scope loads, so no cache write-back or invalidation is
// needed: each wavefront only waits until its own atomics are performed
// before the workgroup arrives.
__device__ inline void row_barrier(int* ws, int P, int phase, int spin_limit) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(ws + kWsBar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int target = phase * P;
    for (int spin = 0; ld_dev(ws + kWsBar) < target; ++spin) {
      if (spin >= spin_limit) {
        __hip_atomic_store(ws + kWsErr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// pick_bucket for a workgroup of kCT threads: nbins / kCT buckets per
// thread, highest at the lowest threads.  Two barriers.
__device__ inline void cpick(const int* hist, int nbins, int r, int above, CShared& sh) {
  const int tid = threadIdx.x;
  const int per = nbins / kCT;   // 16 or 4
  const int top = nbins - per * tid;
  int csum = 0;
  for (int k = 0; k < per; ++k) csum += hist[top - 1 - k];
  int tot;
  const int cum0 = above + block_excl_scan<false, kCWaves>(csum, sh.wsum, &tot);
  if (cum0 < r && cum0 + csum >= r) {
    int cum = cum0, bucket = top - 1;
    for (int k = 0; k < per; ++k) {
      const int ck = hist[top - 1 - k];
      if (cum + ck >= r) {
        bucket = top - 1 - k;
        break;
      }
      cum += ck;
    }
    sh.pick[0] = bucket;
    sh.pick[1] = cum;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kCT) void select_cluster_kernel(SelParams p, int* ws_all, int P, int spin_limit) {
  __shared__ CShared sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / P, seg = blockIdx.x % P;
  int* ws = ws_all + (int64_t)b * cluster_row_ints(P);
  const float* ds = p.ds + (int64_t)b * p.ld;
  const float* ts = p.ts + (int64_t)b * p.ld;
  int32_t* out = p.out + (int64_t)b * p.k_out;
  const int L = p.L;
  const int lo = p.sink < L ? p.sink : L;
  const int w = p.window < L ? p.window : L;
  const int hi = L - w > lo ? L - w : lo;
  const int n_prot = lo + (L - hi);
  const int rest = p.budget - n_prot;
  const int n_free = hi - lo;
  int r1 = p.top_m < rest ? p.top_m : rest;
  r1 = r1 < n_free ? r1 : n_free;
  const int r2 = rest - r1;
  const int j0 = seg * kCSeg + tid * kKPT;

  uint32_t kd[kKPT], kt[kKPT];
  auto load_keys = [&](const float* row, uint32_t (&key)[kKPT]) __attribute__((always_inline)) {
    const bool vec = j0 + kKPT <= L && ((reinterpret_cast<uintptr_t>(row + j0) & 15u) == 0);
    if (vec) {
#pragma unroll
      for (int q = 0; q < kKPT / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(row + j0 + 4 * q);
        key[4 * q + 0] = order_key(v.x);
        key[4 * q + 1] = order_key(v.y);
        key[4 * q + 2] = order_key(v.z);
        key[4 * q + 3] = order_key(v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kKPT; ++i) key[i] = j0 + i < L ? order_key(row[j0 + i]) : 0u;
    }
  };
  load_keys(ds, kd);
  load_keys(ts, kt);
  const uint32_t free = range_bits(j0, lo, hi);
  uint32_t mark = 0;
  int phase = 0;

  // first digit of both tiers; the target histogram counts every free token
  // and is corrected for the draft tier's picks later
  for (int i = tid; i < kBins0; i += kCT) {
    sh.ha[i] = 0;
    sh.hb[i] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKPT; ++i) {
    if ((free >> i) & 1u) {
      if (r1 > 0) atomicAdd(&sh.ha[kd[i] >> kDigitShift[0]], 1);
      if (r2 > 0) atomicAdd(&sh.hb[kt[i] >> kDigitShift[0]], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < kBins0; i += kCT) {
    if (sh.ha[i]) atomicAdd(ws + kWsHd + i, sh.ha[i]);
    if (sh.hb[i]) atomicAdd(ws + kWsHt + i, sh.hb[i]);
  }
  row_barrier(ws, P, ++phase, spin_limit);

  // Marks the top r candidates (free, not yet marked) of tier ti, whose
  // row-wide first-digit histogram is g0.
  auto tier = [&](int ti, int r, const int* g0, uint32_t (&key)[kKPT]) __attribute__((always_inline)) {
    for (int i = tid; i < kBins0; i += kCT) sh.ha[i] = ld_dev(g0 + i);
    __syncthreads();
    cpick(sh.ha, kBins0, r, 0, sh);
    uint32_t prefix = (uint32_t)sh.pick[0] << kDigitShift[0];
    int above = sh.pick[1];
    for (int pass = 1; pass < 3; ++pass) {
      const int shift = kDigitShift[pass];
      const int nb = 1 << kDigitBits[pass];
      const int hs = shift + kDigitBits[pass];   // bits above this digit are fixed
      int* gp = ws + kWsHp + (2 * ti + pass - 1) * 1024;
      for (int i = tid; i < nb; i += kCT) sh.hb[i] = 0;
      __syncthreads();
      const uint32_t cand = free & ~mark;
#pragma unroll
      for (int i = 0; i < kKPT; ++i) {
        if (((cand >> i) & 1u) && (key[i] >> hs) == (prefix >> hs))
          atomicAdd(&sh.hb[(key[i] >> shift) & (uint32_t)(nb - 1)], 1);
      }
      __syncthreads();
      for (int i = tid; i < nb; i += kCT)
        if (sh.hb[i]) atomicAdd(gp + i, sh.hb[i]);
      row_barrier(ws, P, ++phase, spin_limit);
      for (int i = tid; i < nb; i += kCT) sh.ha[i] = ld_dev(gp + i);
      __syncthreads();
      cpick(sh.ha, nb, r, above, sh);
      prefix |= (uint32_t)sh.pick[0] << shift;
      above = sh.pick[1];
    }
    // every candidate above T, and the first (r - above) equal to T in
    // index order over the whole row
    const uint32_t T = prefix;
    const int need_eq = r - above;
    const uint32_t cand = free & ~mark;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kKPT; ++i) {
      const bool c = (cand >> i) & 1u;
      gt |= (uint32_t)(c && key[i] > T) << i;
      eq |= (uint32_t)(c && key[i] == T) << i;
    }
    int tot;
    const int before = block_excl_scan<true, kCWaves>(__popc(eq), sh.wsum, &tot);
    if (tid == 0) __hip_atomic_store(ws + kWsCnt + ti * P + seg, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    row_barrier(ws, P, ++phase, spin_limit);
    int prev = 0;   // equal keys in earlier segments
    for (int q = tid; q < seg; q += kCT) prev += ld_dev(ws + kWsCnt + ti * P + q);
    int earlier;
    block_excl_scan<true, kCWaves>(prev, sh.wsum, &earlier);
    int take = need_eq - earlier - before;
    uint32_t eq_taken = 0;
    for (uint32_t e = eq; e && take > 0; e &= e - 1, --take) eq_taken |= e & (~e + 1u);
    mark |= gt | eq_taken;
  };

  if (r1 > 0) tier(0, r1, ws + kWsHd, kd);
  if (r2 > 0) {
    if (r1 > 0) {
      // take the draft tier's picks out of the target histogram
#pragma unroll
      for (int i = 0; i < kKPT; ++i)
        if ((mark >> i) & 1u) atomicSub(ws + kWsHt + (kt[i] >> kDigitShift[0]), 1);
      row_barrier(ws, P, ++phase, spin_limit);
    }
    tier(1, r2, ws + kWsHt, kt);
  }

  // ascending output: sink, both tiers and window
  const uint32_t valid = range_bits(j0, 0, L);
  const uint32_t sel = (mark | (valid & ~free)) & valid;
  int tot;
  const int before = block_excl_scan<true, kCWaves>(__popc(sel), sh.wsum, &tot);
  if (tid == 0) __hip_atomic_store(ws + kWsCnt + 2 * P + seg, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  row_barrier(ws, P, ++phase, spin_limit);
  int prev = 0;
  for (int q = tid; q < seg; q += kCT) prev += ld_dev(ws + kWsCnt + 2 * P + q);
  int earlier;
  block_excl_scan<true, kCWaves>(prev, sh.wsum, &earlier);
  int pos = earlier + before;
  for (uint32_t e = sel; e; e &= e - 1) {
    const int i = __ffs(e) - 1;
    if (pos < p.k_out) __hip_atomic_store(out + pos, j0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ++pos;
  }
  // The last workgroup of the row to get here sees every other workgroup's
  // output stores performed (agent-scope stores, performed before each
  // workgroup's count): if any wait of the row timed out, the row is
  // replaced by -1.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (tid == 0) sh.pick[0] = __hip_atomic_fetch_add(ws + kWsDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sh.pick[0] == P - 1 && ld_dev(ws + kWsErr) != 0) {
    for (int j = tid; j < p.k_out; j += kCT) __hip_atomic_store(out + j, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(256) void zero_ints_kernel(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// Rows that the multi-workgroup kernel takes: budget < L (checked by the
// caller), longer than one segment of select_kernel (which keeps a
// one-segment row in registers, while longer rows are re-read on every pass;
// a row barrier costs a few microseconds), and every workgroup resident at
// once.  Measured: 16 rows of 32768 tokens 36 us in select_kernel, 53 us
// here (256-thread workgroups); 4 rows of 131072 tokens 178 us there, 58 us
// here (64 us with 256-thread workgroups).
inline int cluster_parts(int32_t B, int32_t L) {
  const int P = (int)(((int64_t)L + kCSeg - 1) / kCSeg);
  return L > kSeg && (int64_t)B * P <= kCMaxGroups ? P : 0;
}

// Workgroups of select_cluster_kernel that the current device holds at once
// (occupancy per CU times CUs; 0 if it cannot be queried), looked up once
// per device.
int cluster_capacity() {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs];   // 0: not looked up yet; else capacity + 1
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kDevs) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c - 1;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)select_cluster_kernel, kCT, 0) !=
          hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int cap = cus * per_cu;
  if (dev >= 0 && dev < kDevs) cache[dev].store(cap + 1, std::memory_order_relaxed);
  return cap;
}

// Polls per row-barrier wait: kSpinLimit, or VA_SELECT_SPIN_LIMIT from the
// environment (a test hook: a limit of 0 makes every early arrival give up
// at once, which exercises the timeout path).
int spin_limit() {
  const char* e = getenv("VA_SELECT_SPIN_LIMIT");
  if (e == nullptr || *e == '\0') return kSpinLimit;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? 0 : (v > kSpinLimit ? kSpinLimit : (int)v);
}

}  // namespace

size_t select_ws_bytes(int32_t B, int32_t L) {
  const int P = cluster_parts(B, L);
  return P ? (size_t)B * cluster_row_ints(P) * sizeof(int) : 0;
}

hipError_t launch_select(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                         int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                         void* ws, hipStream_t stream) {
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
  int P = budget < L ? cluster_parts(B, L) : 0;
  if (P && cluster_capacity() < B * P) P = 0;   // not every workgroup would be resident
  if (P) {
    const int64_t n = (int64_t)B * cluster_row_ints(P);
    const int grid = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(zero_ints_kernel, dim3(grid), dim3(256), 0, stream, (int*)ws, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int* ws_i = (int*)ws;
    int lim = spin_limit();
    // (a cooperative launch, which would have the runtime guarantee
    // co-residency, cost ~20 us per call: 56 -> 76 us on 4 rows of 131072)
    hipLaunchKernelGGL(select_cluster_kernel, dim3(B * P), dim3(kCT), 0, stream, p, ws_i, P, lim);
    return hipGetLastError();
  }
  const int nseg = (L + kSeg - 1) / kSeg;
  const size_t lds = (size_t)(nseg > 0 ? nseg : 1) * kST * sizeof(uint32_t);
  const bool resident = nseg <= 1;
  const void* fn = resident ? (const void*)select_kernel<true> : (const void*)select_kernel<false>;
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (resident)
    hipLaunchKernelGGL(select_kernel<true>, dim3(B), dim3(kST), lds, stream, p);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3(B), dim3(kST), lds, stream, p);
  return hipGetLastError();
}

}  // namespace va
