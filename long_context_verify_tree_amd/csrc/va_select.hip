// Verify-set selection for sparse verification (Dustin, "Aggregazione
// Ibrida dell'Attenzione"): keep the attention-sink prefix and the local
// window, take the top-m tokens by draft-lookahead score, then fill the rest
// of the budget with the best remaining tokens by target-historical score.
//
// Each tier is an exact top-r over its candidates (the free tokens between
// sink and window; for the target tier, minus the draft tier's picks), ties
// going to the lower index.  Scores become order-preserving 32-bit keys (NaN
// lowest, -0 == +0) and a token's rank is the 64-bit value (key << 32) |
// ~index: higher is better, and no two tokens share one.  A tier's result is
// one threshold P, the rank of its r-th best candidate; the tier takes
// exactly the candidates whose rank is >= P.
//
// Two kernels per call, with no waits between workgroups:
//   * select_filter_kernel, many 4096-token workgroups per row.  Every
//     workgroup of a row reads the same row-wide sample (one 32-token run per
//     block of the row, at most 128 blocks) and derives from it, for each
//     tier, a key bound K below which the tier surely does not reach: the
//     top-12-bit bucket of sample rank r f + 4 sqrt(r f) + 4 (f the sample's
//     share of the free tokens; for the target tier the sample leaves out
//     the tokens at or above the draft bound, a superset of the draft picks,
//     which can only lower K).  It then writes, in index order, every free
//     token of its segment with a draft key >= K_d or a target key >= K_t
//     (both keys and the index) to its own region of the workspace.
//   * select_resolve_kernel, one 1024-thread workgroup per row, gathers the
//     regions into LDS, still in index order.  If the draft tier has at least
//     r1 listed candidates and the target tier (listed tokens below the draft
//     threshold with a target key >= K_t) at least r2, every token a tier
//     could take is listed, and each threshold is found among the listed
//     entries alone: radix passes (12, 10 and 10 bits) of LDS histograms
//     until the bin of the r-th best holds at most 64 entries, whose ranks
//     are then compared with one another, or, after the last pass, an
//     index-order scan of the entries equal to the threshold key.  The
//     output (sink, the listed entries at or above their tier's threshold,
//     window) follows from one scan of the list.  Otherwise (a sample far
//     off, a full region or list) the same workgroup takes the exact way
//     over the whole row: the same radix passes over every key, re-read from
//     the row per pass, and an index-order scan of the threshold key's ties.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "va_device.h"
#include "va_select.h"

namespace va {
namespace {

constexpr int kBins = 4096;               // buckets of a key's top 12 bits
constexpr int kTiny = 64;                 // entries of the last bin compared pairwise
constexpr uint64_t kNone = ~0ull;         // threshold that takes no token
constexpr uint32_t kNoKey = 0xFFFFFFFFu;  // key bound that lists no token (keys are <= 0xFF800000)

struct SelParams {
  const float* ds;
  const float* ts;
  int32_t* out;
  int64_t ld;
  int L, budget, k_out;
  int lo, hi, n_free, r1, r2;   // free tokens [lo, hi); picks of the two tiers
  int exact;                    // take the exact way only (a test hook)
};

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;               // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;        // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint32_t key_of_bits(uint32_t bits) { return order_key(__uint_as_float(bits)); }

__device__ inline uint64_t rank_of(uint32_t key, int j) { return ((uint64_t)key << 32) | (uint32_t)~(uint32_t)j; }

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

// Exclusive prefix sum of v over the workgroup (NW wavefronts) in thread
// order; *total gets the sum.  One barrier, plus a second with TAIL for a
// caller that writes wsum again before its next barrier.
template <bool TAIL, int NW>
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

// Bits of the four tokens [b, b + 4) that lie in [lo, hi).
__device__ inline uint32_t nib_bits(int b, int lo, int hi) {
  int a = lo - b, e = hi - b;
  a = a < 0 ? 0 : (a > 4 ? 4 : a);
  e = e < 0 ? 0 : (e > 4 ? 4 : e);
  return ((1u << e) - 1u) & ~((1u << a) - 1u);
}

// Counts of a histogram of NB buckets split over NT threads (NB / NT each,
// the highest buckets at the lowest threads): c[] gets this thread's counts,
// highest first; returns the count in higher buckets and *total the sum.
// One barrier; the caller reaches another before wsum is written again.
template <int NT, int NB>
__device__ inline int bins_scan(const int* hist, int (&c)[NB / NT], int* wsum, int* total) {
  constexpr int PER = NB / NT;
  const int top = NB - PER * (int)threadIdx.x;
  int csum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    c[k] = hist[top - 1 - k];
    csum += c[k];
  }
  return block_excl_scan<false, NT / 64>(csum, wsum, total);
}

// If the rank-th largest entry (1-based) lies in this thread's buckets
// (cum entries in higher ones), returns its bucket and sets *above to the
// entries in higher buckets; else -1.
template <int NT, int NB>
__device__ inline int bins_find(const int (&c)[NB / NT], int cum, int rank, int* above, int* count = nullptr) {
  constexpr int PER = NB / NT;
  const int top = NB - PER * (int)threadIdx.x;
  if (rank <= cum) return -1;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (rank <= cum + c[k]) {
      *above = cum;
      if (count) *count = c[k];
      return top - 1 - k;
    }
    cum += c[k];
  }
  return -1;
}

// Radix digits of a key: 12 bits, then 10, then 10.
__device__ inline int digit_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 10 : 0); }
__device__ inline int digit_bins(int pass) { return pass == 0 ? kBins : 1024; }

// ---------------------------------------------------------------------------
// The filter: 512 threads, 8 tokens each (two runs of four), per 4096-token
// segment.  Thread t holds tokens base + 2048 q + 4 t + e (q < 2, e < 4) as
// bit 4 q + e, so each load of four tokens is coalesced across the
// wavefront and index order is (q, t, e).

constexpr int kFT = 512;                   // threads per filter workgroup
constexpr int kFW = kFT / 64;
constexpr int kFSeg = 8 * kFT;             // tokens per filter workgroup
constexpr int kFCap = kFSeg / 2;           // entries a segment may list
constexpr int kSampBlocks = 128;           // row-wide sample: at most this many 32-token runs
constexpr int kSampPT = kSampBlocks * 32 / kFT;   // sample tokens per thread (8)
constexpr int kMaxFP = (kSelectMaxL + kFSeg - 1) / kFSeg;   // segments of the longest row
static_assert(kSampPT == 8, "two runs of four sample tokens per thread");

// Workspace of one row, in ints: the two key bounds, the segments' list
// counts, then per segment its listed draft keys, target keys and indices.
constexpr int kWsKd = 0;
constexpr int kWsKt = 1;
constexpr int kWsCnt = 64;
constexpr int kWsReg = kWsCnt + (kMaxFP + 63) / 64 * 64;
constexpr int kRegInts = 3 * kFCap;

__host__ __device__ inline int filter_parts(int L) { return (L + kFSeg - 1) / kFSeg; }
__host__ __device__ inline int64_t row_ints(int L) { return kWsReg + (int64_t)filter_parts(L) * kRegInts; }

struct FShared {
  int hs[kBins];
  int wsum[kFW];
  int pick;
};

// Key bound of a tier from the sample histogram sh.hs: the bucket holding
// sample rank ceil(r f + 4 sqrt(r f) + 4), f = S / n_free (S < 0: the
// histogram's own total), shifted to a key; 0 when the sample holds fewer.
// *total gets the histogram's total.  Two barriers.
__device__ inline uint32_t key_bound(int r, int S, int n_free, FShared& sh, int* total) {
  int c[kBins / kFT], tot;
  if (threadIdx.x == 0) sh.pick = 0;
  const int cum = bins_scan<kFT, kBins>(sh.hs, c, sh.wsum, &tot);
  const float fe = (float)r * (float)(S < 0 ? tot : S) / (float)n_free;
  const int rank = (int)ceilf(fe + 4.0f * sqrtf(fe) + 4.0f);
  int ab;
  const int bk = bins_find<kFT, kBins>(c, cum, rank, &ab);
  if (bk >= 0) sh.pick = bk;
  __syncthreads();
  *total = tot;
  return (uint32_t)sh.pick << 20;
}

__global__ __launch_bounds__(kFT) void select_filter_kernel(SelParams p, int* ws_all, int P) {
  __shared__ FShared sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / P, seg = blockIdx.x % P;
  const int base = seg * kFSeg;
  int* ws = ws_all + (int64_t)b * row_ints(p.L);
  const float* ds = p.ds + (int64_t)b * p.ld;
  const float* ts = p.ts + (int64_t)b * p.ld;
  const int L = p.L, lo = p.lo, hi = p.hi;

  // this segment's scores (raw bits first, so that every load is in flight
  // at once), then the row-wide sample: block k of nblk (each sb tokens)
  // contributes the 32-token run at 32 * (7 k mod sb / 32) past its start;
  // this thread takes tokens u .. u + 3 of the runs for u = 4 t, 4 t + 2048
  uint32_t kd[8], kt[8];
  const int b0 = base + 4 * tid;
  const bool aligned = ((reinterpret_cast<uintptr_t>(ds) | reinterpret_cast<uintptr_t>(ts)) & 15u) == 0;
  const dev::rsrc_t rsd = dev::make_rsrc(ds, (uint32_t)L * 4u), rst = dev::make_rsrc(ts, (uint32_t)L * 4u);
  if (aligned && base + kFSeg <= L) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 a = *reinterpret_cast<const uint4*>(ds + b0 + q * 4 * kFT);
      const uint4 c = *reinterpret_cast<const uint4*>(ts + b0 + q * 4 * kFT);
      kd[4 * q + 0] = a.x, kd[4 * q + 1] = a.y, kd[4 * q + 2] = a.z, kd[4 * q + 3] = a.w;
      kt[4 * q + 0] = c.x, kt[4 * q + 1] = c.y, kt[4 * q + 2] = c.z, kt[4 * q + 3] = c.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = b0 + (i >> 2) * 4 * kFT + (i & 3);   // (past L: reads 0, never listed)
      kd[i] = __builtin_amdgcn_raw_buffer_load_b32(rsd, j * 4, 0, 0);
      kt[i] = __builtin_amdgcn_raw_buffer_load_b32(rst, j * 4, 0, 0);
    }
  }
  const int nblk0 = (L + 255) / 256;
  const int nblk = nblk0 < kSampBlocks ? nblk0 : kSampBlocks;
  const int sb = (L + 32 * nblk - 1) / (32 * nblk) * 32;
  uint32_t sd[kSampPT], st[kSampPT];
  int sj[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = 4 * tid + h * 4 * kFT;
    const int k = u >> 5;
    const int j = k * sb + 32 * ((7 * k) % (sb / 32)) + (u & 31);
    sj[h] = k < nblk ? j : L;
    if (aligned && k < nblk && j + 4 <= L) {
      const uint4 a = *reinterpret_cast<const uint4*>(ds + j);
      const uint4 c = *reinterpret_cast<const uint4*>(ts + j);
      sd[4 * h + 0] = a.x, sd[4 * h + 1] = a.y, sd[4 * h + 2] = a.z, sd[4 * h + 3] = a.w;
      st[4 * h + 0] = c.x, st[4 * h + 1] = c.y, st[4 * h + 2] = c.z, st[4 * h + 3] = c.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sd[4 * h + e] = __builtin_amdgcn_raw_buffer_load_b32(rsd, (sj[h] + e) * 4, 0, 0);
        st[4 * h + e] = __builtin_amdgcn_raw_buffer_load_b32(rst, (sj[h] + e) * 4, 0, 0);
      }
    }
  }
  for (int i = tid; i < kBins; i += kFT) sh.hs[i] = 0;
  uint32_t sfree = 0;   // sample tokens that are free
#pragma unroll
  for (int k = 0; k < kSampPT; ++k) {
    const int j = sj[k >> 2] + (k & 3);
    sfree |= (uint32_t)(j >= lo && j < hi) << k;
    sd[k] = key_of_bits(sd[k]);
  }
  __syncthreads();

  // the key bounds of the two tiers
  uint32_t K_d = kNoKey, K_t = kNoKey;
  int S = 0;   // free sample tokens
  if (p.r1 > 0) {
#pragma unroll
    for (int k = 0; k < kSampPT; ++k)
      if ((sfree >> k) & 1u) atomicAdd(&sh.hs[sd[k] >> 20], 1);
    __syncthreads();
    K_d = key_bound(p.r1, -1, p.n_free, sh, &S);
    for (int i = tid; i < kBins; i += kFT) sh.hs[i] = 0;
    __syncthreads();
  } else {
    block_excl_scan<true, kFW>(__popc(sfree), sh.wsum, &S);
  }
  if (p.r2 > 0) {
#pragma unroll
    for (int k = 0; k < kSampPT; ++k)
      if (((sfree >> k) & 1u) && sd[k] < K_d) atomicAdd(&sh.hs[key_of_bits(st[k]) >> 20], 1);
    __syncthreads();
    int t2;
    K_t = key_bound(p.r2, S, p.n_free, sh, &t2);
  }
  if (seg == 0 && tid == 0) {
    ws[kWsKd] = (int)K_d;
    ws[kWsKt] = (int)K_t;
  }

  // list, in index order, the free tokens either tier could take
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    kd[i] = key_of_bits(kd[i]);
    kt[i] = key_of_bits(kt[i]);
    const int j = b0 + (i >> 2) * 4 * kFT + (i & 3);
    keep |= (uint32_t)(j >= lo && j < hi && (kd[i] >= K_d || kt[i] >= K_t)) << i;
  }
  const int v = __popc(keep & 15u) | (__popc(keep >> 4) << 16);
  int tot;
  const int ex = block_excl_scan<false, kFW>(v, sh.wsum, &tot);
  const int n0 = tot & 0xffff, n = n0 + (tot >> 16);
  int* reg = ws + kWsReg + (int64_t)seg * kRegInts;
  int pos0 = ex & 0xffff, pos1 = n0 + (ex >> 16);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((keep >> i) & 1u) {
      const int at = i < 4 ? pos0++ : pos1++;
      if (at < kFCap) {
        reg[at] = (int)kd[i];
        reg[kFCap + at] = (int)kt[i];
        reg[2 * kFCap + at] = b0 + (i >> 2) * 4 * kFT + (i & 3);
      }
    }
  }
  if (tid == 0) ws[kWsCnt + seg] = n;
}

// ---------------------------------------------------------------------------
// The resolve: one workgroup of 1024 threads per row.

constexpr int kRT = 1024;                  // threads per resolve workgroup
constexpr int kRW = kRT / 64;
constexpr int kRCap = 8192;                // list entries resolved in LDS
constexpr int kEPT = kRCap / kRT;          // list entries per thread at most (8)
// The exact way walks a row in segments of kXQ runs of 4096 tokens (kXQ * 4
// keys per thread).  Four runs: 16 keys per thread, so that the fallback's
// registers stay below what the list path needs and the kernel needs no
// scratch (with eight runs, 32 keys and another 32 for the target tier's
// draft picks, it spilled and every call paid for it, taken or not).
constexpr int kXQ = 4;
constexpr int kXK = 4 * kXQ;               // keys per thread per exact-way segment
constexpr int kSeg = kRT * kXK;            // tokens per exact-way segment
static_assert(kSelectSegTokens % kSeg == 0, "the length limit is whole exact-way segments");
static_assert(kMaxFP <= kRT, "one segment count per thread");

struct RShared {
  union {
    struct {
      uint32_t kd[kRCap];
      uint32_t kt[kRCap];
      int j[kRCap];
    } e;                      // the row's list, in index order
    int off[kMaxFP];          // (segment offsets, before the list is read)
  } u;
  int h0[2][kBins];           // top 12 bits, one histogram per tier
  int h1[1024];               // next 10 bits
  int h2[1024];               // last 10 bits
  uint64_t tiny[kTiny];
  int wsum[kRW];
  int pick[3];
  int ntiny;
  uint64_t pstar;
};

// Threshold of the r-th best among the list entries of this thread's span
// [e0, e0 + cnt) whose bit is set in cand (bit e - e0), by key (the kd or kt
// list).  Radix passes until the r-th best's bin holds at most kTiny
// entries (then compared pairwise), else an index-order scan of its ties
// after the last pass.
__device__ __forceinline__ uint64_t list_select(const uint32_t* key, const int* jj, int e0, int cnt, uint32_t cand, int r,
                                int* h0, RShared& sh, bool* ok) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, fixed = 0;   // key bits found so far, and their mask
  int above = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass), nb = digit_bins(pass);
    int* hist = pass == 0 ? h0 : (pass == 1 ? sh.h1 : sh.h2);
#pragma unroll
    for (int k = 0; k < kEPT; ++k) {
      if (k < cnt && ((cand >> k) & 1u)) {
        const uint32_t kv = key[e0 + k];
        if ((kv & fixed) == prefix) atomicAdd(&hist[(kv >> shift) & (uint32_t)(nb - 1)], 1);
      }
    }
    if (pass < 2) {   // the next pass's histogram
      int* next = pass == 0 ? sh.h1 : sh.h2;
      for (int i = tid; i < 1024; i += kRT) next[i] = 0;
    }
    if (tid == 0) sh.ntiny = 0;
    __syncthreads();
    int bk = -1, ab = 0, bc = 0, t0 = 0;
    if (pass == 0) {
      int c[kBins / kRT];
      const int cum = above + bins_scan<kRT, kBins>(hist, c, sh.wsum, &t0);
      bk = bins_find<kRT, kBins>(c, cum, r, &ab, &bc);
    } else {
      int c[1024 / kRT], t;
      const int cum = above + bins_scan<kRT, 1024>(hist, c, sh.wsum, &t);
      bk = bins_find<kRT, 1024>(c, cum, r, &ab, &bc);
    }
    if (bk >= 0) {
      sh.pick[0] = bk;
      sh.pick[1] = ab;
      sh.pick[2] = bc;
    }
    __syncthreads();
    if (pass == 0 && t0 < r) {   // fewer candidates than picks (t0: every candidate; uniform)
      *ok = false;
      return kNone;
    }
    prefix |= (uint32_t)sh.pick[0] << shift;
    fixed |= (uint32_t)(nb - 1) << shift;
    above = sh.pick[1];
    const int E = sh.pick[2];
    if (E <= kTiny) {
      // the bin's entries, compared pairwise
#pragma unroll
      for (int k = 0; k < kEPT; ++k) {
        if (k < cnt && ((cand >> k) & 1u)) {
          const uint32_t kv = key[e0 + k];
          if ((kv & fixed) == prefix) {
            const int s = atomicAdd(&sh.ntiny, 1);
            if (s < kTiny) sh.tiny[s] = rank_of(kv, jj[e0 + k]);
          }
        }
      }
      __syncthreads();
      if (tid < E) {
        const uint64_t rv = sh.tiny[tid];
        int rk = 0;
        for (int x = 0; x < E; ++x) rk += sh.tiny[x] > rv;
        if (rk == r - above - 1) sh.pstar = rv;
      }
      __syncthreads();
      return sh.pstar;
    }
  }
  // more than kTiny entries share the key T = prefix: the (r - above)-th of
  // them in list (index) order is the last taken
  int eq = 0;
#pragma unroll
  for (int k = 0; k < kEPT; ++k) eq += (k < cnt && ((cand >> k) & 1u) && key[e0 + k] == prefix) ? 1 : 0;
  int tot;
  int before = block_excl_scan<true, kRW>(eq, sh.wsum, &tot);
  const int need = r - above;
#pragma unroll
  for (int k = 0; k < kEPT; ++k) {
    if (k < cnt && ((cand >> k) & 1u) && key[e0 + k] == prefix) {
      if (++before == need) sh.pstar = rank_of(prefix, jj[e0 + k]);
    }
  }
  __syncthreads();
  return sh.pstar;
}

// The exact way.  A segment of kSeg tokens: thread t holds tokens
// base + 4096 q + 4 t + e (q < kXQ, e < 4) as bit 4 q + e; index order is
// (q, t, e).  Tokens past L read 0 (never candidates).
__device__ inline void seg_keys(dev::rsrc_t rs, bool vec, const float* row, int base, uint32_t (&key)[kXK]) {
  const int b0 = base + 4 * (int)threadIdx.x;
  if (vec) {
#pragma unroll
    for (int q = 0; q < kXQ; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + b0 + q * 4 * kRT);
      key[4 * q + 0] = v.x, key[4 * q + 1] = v.y, key[4 * q + 2] = v.z, key[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kXK; ++i)
      key[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (b0 + (i >> 2) * 4 * kRT + (i & 3)) * 4, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kXK; ++i) key[i] = key_of_bits(key[i]);
}

__device__ inline int seg_token(int base, int i) { return base + (i >> 2) * 4 * kRT + 4 * (int)threadIdx.x + (i & 3); }

__device__ inline uint32_t seg_bits(int base, int lo, int hi) {
  const int b0 = base + 4 * (int)threadIdx.x;
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < kXQ; ++q) m |= nib_bits(b0 + q * 4 * kRT, lo, hi) << (4 * q);
  return m;
}

// Bits of this thread's tokens whose rank is >= P.
__device__ inline uint32_t seg_sel(const uint32_t (&key)[kXK], int base, uint64_t P) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kXK; ++i) m |= (uint32_t)(rank_of(key[i], seg_token(base, i)) >= P) << i;
  return m;
}

// The exact way for one tier over the whole row: threshold of the r-th best
// candidate by the keys of `row` (for the target tier, the draft picks, rank
// >= pd by the keys of drow, are not candidates).
__device__ uint64_t exact_tier(const SelParams p, const float* row, const float* drow, uint64_t pd, bool target,
                               int r, RShared& sh) {
  const int tid = threadIdx.x;
  const int L = p.L, nseg = (L + kSeg - 1) / kSeg;
  const dev::rsrc_t rs = dev::make_rsrc(row, (uint32_t)L * 4u), rsd = dev::make_rsrc(drow, (uint32_t)L * 4u);
  const bool al = ((reinterpret_cast<uintptr_t>(row) | reinterpret_cast<uintptr_t>(drow)) & 15u) == 0;
  uint32_t key[kXK];
  auto cand_of = [&](int s) __attribute__((always_inline)) {
    uint32_t c = seg_bits(s * kSeg, p.lo, p.hi);
    if (target) {
      uint32_t k2[kXK];
      seg_keys(rsd, al && (s + 1) * kSeg <= L, drow, s * kSeg, k2);
      c &= ~seg_sel(k2, s * kSeg, pd);
    }
    return c;
  };
  uint32_t prefix = 0, fixed = 0;
  int above = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass), nb = digit_bins(pass);
    int* hist = pass == 0 ? sh.h0[0] : sh.h1;
    for (int i = tid; i < nb; i += kRT) hist[i] = 0;
    __syncthreads();
    for (int s = 0; s < nseg; ++s) {
      const uint32_t cand = cand_of(s);
      seg_keys(rs, al && (s + 1) * kSeg <= L, row, s * kSeg, key);
#pragma unroll
      for (int i = 0; i < kXK; ++i)
        if (((cand >> i) & 1u) && (key[i] & fixed) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & (uint32_t)(nb - 1)], 1);
    }
    __syncthreads();
    int bk = -1, ab = 0;
    if (pass == 0) {
      int c[kBins / kRT], t;
      const int cum = above + bins_scan<kRT, kBins>(hist, c, sh.wsum, &t);
      bk = bins_find<kRT, kBins>(c, cum, r, &ab);
    } else {
      int c[1024 / kRT], t;
      const int cum = above + bins_scan<kRT, 1024>(hist, c, sh.wsum, &t);
      bk = bins_find<kRT, 1024>(c, cum, r, &ab);
    }
    if (bk >= 0) {
      sh.pick[0] = bk;
      sh.pick[1] = ab;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.pick[0] << shift;
    fixed |= (uint32_t)(nb - 1) << shift;
    above = sh.pick[1];
    __syncthreads();   // (every thread has read the pick)
  }
  // the (r - above)-th candidate equal to T in index order is the last taken
  const int need = r - above;
  int run = 0;
  for (int s = 0; s < nseg; ++s) {
    const uint32_t cand = cand_of(s);
    seg_keys(rs, al && (s + 1) * kSeg <= L, row, s * kSeg, key);
    uint32_t eq = 0;
#pragma unroll
    for (int i = 0; i < kXK; ++i) eq |= (uint32_t)(((cand >> i) & 1u) && key[i] == prefix) << i;
    for (int q = 0; q < kXQ; ++q) {   // one scan per run of 4096 tokens
      const uint32_t nbits = (eq >> (4 * q)) & 15u;
      int tot;
      int before = run + block_excl_scan<true, kRW>(__popc(nbits), sh.wsum, &tot);
      for (int e = 0; e < 4; ++e) {
        if ((nbits >> e) & 1u) {
          if (++before == need) sh.pstar = rank_of(prefix, seg_token(s * kSeg, 4 * q + e));
        }
      }
      run += tot;
    }
  }
  __syncthreads();
  return sh.pstar;
}

// Output of the exact way: sink, the tiers' picks and window, ascending.
__device__ void exact_output(const SelParams p, const float* ds, const float* ts, int32_t* out, uint64_t pd,
                             uint64_t pt, RShared& sh) {
  const int L = p.L, nseg = (L + kSeg - 1) / kSeg;
  const dev::rsrc_t rsd = dev::make_rsrc(ds, (uint32_t)L * 4u), rst = dev::make_rsrc(ts, (uint32_t)L * 4u);
  const bool al = ((reinterpret_cast<uintptr_t>(ds) | reinterpret_cast<uintptr_t>(ts)) & 15u) == 0;
  int written = 0;
  for (int s = 0; s < nseg; ++s) {
    uint32_t key[kXK];
    const bool vec = al && (s + 1) * kSeg <= L;
    const uint32_t f = seg_bits(s * kSeg, p.lo, p.hi), valid = seg_bits(s * kSeg, 0, L);
    seg_keys(rsd, vec, ds, s * kSeg, key);
    const uint32_t dsel = f & seg_sel(key, s * kSeg, pd);
    seg_keys(rst, vec, ts, s * kSeg, key);
    const uint32_t sel = (valid & ~f) | dsel | (f & ~dsel & seg_sel(key, s * kSeg, pt));
    for (int q = 0; q < kXQ; ++q) {
      const uint32_t nbits = (sel >> (4 * q)) & 15u;
      int tot;
      int pos = written + block_excl_scan<true, kRW>(__popc(nbits), sh.wsum, &tot);
      for (int e = 0; e < 4; ++e) {
        if ((nbits >> e) & 1u) {
          if (pos < p.k_out) out[pos] = seg_token(s * kSeg, 4 * q + e);
          ++pos;
        }
      }
      written += tot;
    }
  }
}

__global__ __launch_bounds__(kRT) void select_resolve_kernel(SelParams p, const int* ws_all, int P) {
  __shared__ RShared sh;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const float* ds = p.ds + (int64_t)b * p.ld;
  const float* ts = p.ts + (int64_t)b * p.ld;
  int32_t* out = p.out + (int64_t)b * p.k_out;
  const int L = p.L, lo = p.lo, hi = p.hi, r1 = p.r1, r2 = p.r2;
  if (p.budget >= L) {
    for (int j = tid; j < L; j += kRT) out[j] = j;
    return;
  }
  uint64_t pd = kNone, pt = kNone;
  if (!p.exact) {
    const int* ws = ws_all + (int64_t)b * row_ints(L);
    // segment offsets of the list (a count past kFCap marks a full region)
    const int c = tid < P ? ws[kWsCnt + tid] : 0;
    int tot;
    const int off = block_excl_scan<true, kRW>(c + (c > kFCap ? (1 << 20) : 0), sh.wsum, &tot);
    const int n = tot & ((1 << 20) - 1);
    bool ok = (tot >> 20) == 0 && n <= kRCap;
    if (ok) {
      // gather the regions into LDS in index order, G threads per region
      if (tid < P) sh.u.off[tid] = off;
      for (int i = tid; i < kBins; i += kRT) {
        sh.h0[0][i] = 0;
        sh.h0[1][i] = 0;
      }
      __syncthreads();
      const int G = kRT / P;
      const int s = tid / G, lt = tid % G;
      int so = 0, sc = 0;
      if (s < P) {
        so = sh.u.off[s];
        sc = (s + 1 < P ? sh.u.off[s + 1] : n) - so;
      }
      __syncthreads();
      if (s < P) {
        const int* reg = ws + kWsReg + (int64_t)s * kRegInts;
        for (int i0 = lt; i0 < sc; i0 += 4 * G) {   // four entries in flight
          uint32_t a[4], t[4];
          int jj[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * G < sc ? i0 + u * G : i0;
            a[u] = (uint32_t)reg[i];
            t[u] = (uint32_t)reg[kFCap + i];
            jj[u] = reg[2 * kFCap + i];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (i0 + u * G < sc) {
              sh.u.e.kd[so + i0 + u * G] = a[u];
              sh.u.e.kt[so + i0 + u * G] = t[u];
              sh.u.e.j[so + i0 + u * G] = jj[u];
            }
          }
        }
      }
      __syncthreads();
      // this thread's span of the list
      const int per = (n + kRT - 1) / kRT;
      const int e0 = tid * per;
      const int cnt = e0 < n ? (n - e0 < per ? n - e0 : per) : 0;
      const uint32_t K_d = (uint32_t)ws[kWsKd], K_t = (uint32_t)ws[kWsKt];
      uint32_t cd = 0;
#pragma unroll
      for (int k = 0; k < kEPT; ++k) cd |= (uint32_t)(k < cnt && sh.u.e.kd[e0 + k] >= K_d) << k;
      if (r1 > 0) pd = list_select(sh.u.e.kd, sh.u.e.j, e0, cnt, cd, r1, sh.h0[0], sh, &ok);
      uint32_t ct = 0;
      if (ok) {
#pragma unroll
        for (int k = 0; k < kEPT; ++k)
          ct |= (uint32_t)(k < cnt && rank_of(sh.u.e.kd[e0 + k], sh.u.e.j[e0 + k]) < pd && sh.u.e.kt[e0 + k] >= K_t)
                << k;
        if (r2 > 0) pt = list_select(sh.u.e.kt, sh.u.e.j, e0, cnt, ct, r2, sh.h0[1], sh, &ok);
      }
      if (ok) {
        // sink, the listed picks in index order, window
        uint32_t win = 0;
#pragma unroll
        for (int k = 0; k < kEPT; ++k) {
          if (k < cnt) {
            const bool d = rank_of(sh.u.e.kd[e0 + k], sh.u.e.j[e0 + k]) >= pd;
            const bool t = ((ct >> k) & 1u) && rank_of(sh.u.e.kt[e0 + k], sh.u.e.j[e0 + k]) >= pt;
            win |= (uint32_t)(d || t) << k;
          }
        }
        int tw;
        int pos = lo + block_excl_scan<true, kRW>(__popc(win), sh.wsum, &tw);
#pragma unroll
        for (int k = 0; k < kEPT; ++k)
          if (((win >> k) & 1u) && pos < p.k_out) out[pos++] = sh.u.e.j[e0 + k];
        for (int j = tid; j < lo; j += kRT) out[j] = j;
        for (int j = tid; j < L - hi; j += kRT) out[lo + r1 + r2 + j] = hi + j;
        return;
      }
    }
    __syncthreads();
    pd = kNone;
    pt = kNone;
  }
  // the exact way over the whole row
  if (r1 > 0) pd = exact_tier(p, ds, ds, kNone, false, r1, sh);
  if (r2 > 0) pt = exact_tier(p, ts, ds, pd, true, r2, sh);
  exact_output(p, ds, ts, out, pd, pt, sh);
}

// VA_SELECT_EXACT=1 in the environment makes every call take the exact way
// (a test hook: both ways must give the same verify set).
int exact_only() {
  const char* e = getenv("VA_SELECT_EXACT");
  return e != nullptr && e[0] == '1';
}

}  // namespace

size_t select_ws_bytes(int32_t B, int32_t L) { return (size_t)B * (size_t)row_ints(L) * sizeof(int); }

hipError_t launch_select(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                         int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                         void* ws, hipStream_t stream) {
  SelParams p{};
  p.ds = draft_score;
  p.ts = target_score;
  p.out = verify_idx;
  p.ld = ld;
  p.L = L;
  p.budget = budget;
  p.k_out = budget < L ? budget : L;
  p.lo = sink < L ? sink : L;
  const int w = window < L ? window : L;
  p.hi = L - w > p.lo ? L - w : p.lo;
  p.n_free = p.hi - p.lo;
  const int rest = budget - (p.lo + (L - p.hi));
  const int r1 = top_m < rest ? top_m : rest;
  p.r1 = r1 < p.n_free ? r1 : p.n_free;
  p.r2 = rest - p.r1;
  p.exact = exact_only();
  const int P = filter_parts(L);
  if (budget < L && !p.exact) {
    hipLaunchKernelGGL(select_filter_kernel, dim3(B * P), dim3(kFT), 0, stream, p, (int*)ws, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_resolve_kernel, dim3(B), dim3(kRT), 0, stream, p, (const int*)ws, P);
  return hipGetLastError();
}

}  // namespace va
