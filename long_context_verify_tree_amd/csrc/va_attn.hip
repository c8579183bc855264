// Verification-attention kernels for gfx950 (MI355X).
//
// The hybrid tree attention of LongSpec ("Tree Attention Ibrida") splits the
// target model's verification attention into an unmasked context part over
// the KV cache and a tree-masked part over the draft tokens, and joins the
// two with a log-sum-exp merge.  Here the context part is further split
// along the keys (split-K flash decoding) so that a single long sequence
// spreads over the whole chip:
//
//   partial_kernel  one workgroup per (sequence, kv head, row tile, part).
//                   Parts 0..S-1 are context splits (dense range or gathered
//                   verify-set indices, Dustin "Workflow di Verifica");
//                   part S is the draft tree under its ancestor mask (in a
//                   dense call whose context workgroups fill the chip, the
//                   last context split walks the tree after its context
//                   keys instead).
//                   Writes a normalised partial row and its log2-sum-exp.
//   merge_kernel    D / 4 lanes per output row (16 bytes of each part per
//                   lane): log-sum-exp merge of the row's partials.
//
// Inside partial_kernel the four wavefronts of a workgroup stream disjoint
// 32-key tiles (wave w takes tiles w, w+4, ...).  Each tile of K and V is
// fetched with coalesced 16-byte loads one tile ahead into registers, staged
// in a wave-private LDS tile and fed to MFMA:
//   S^T[32 keys x 32 rows] = K_tile . Q^T   (v_mfma_f32_32x32x16_bf16, or
//                                            v_mfma_f32_32x32x2f32 for fp32)
//   O^T[D x 32 rows]      += V_tile^T . P^T
// with an online softmax in fp32 (exp2, scale*log2(e) folded into one FMA).
// P^T is used as the MFMA B operand straight from the S^T accumulator
// layout: the contraction index of the PV product is relabelled to match it,
// so no cross-lane movement of P is needed; only V is read transposed from
// LDS.  The four wavefronts' running (max, sum, O) are merged in LDS in a
// fixed order, so results are bitwise reproducible.

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "va_device.h"
#include "va_internal.h"

namespace va {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 32;
constexpr int kMaxN = 256;
constexpr int kAncWords = kMaxN / 32;

#ifndef VA_ROTATE
#define VA_ROTATE 1   // per-head start offset of the context tile walk
#endif
#ifndef VA_TREE_FIRST
#define VA_TREE_FIRST 1
#endif
// Work item of this workgroup: (row tile, part, kv head, sequence).
// The draft-tree parts are short; with VA_TREE_FIRST they take the lowest
// workgroup ids, which are dispatched first, so no long context part waits
// behind them.  Context parts are mapped XCD-aware among themselves.
__device__ inline void decode_group(const PartialParams& p, int& rt, int& part, int& kvh, int& b) {
  int id;
  if (VA_TREE_FIRST) {
    const int ntree = p.tree_in_last ? 0 : p.B * p.Hkv * p.row_tiles;
    if ((int)blockIdx.x < ntree) {
      id = blockIdx.x;
      rt = id % p.row_tiles;
      id /= p.row_tiles;
      part = p.n_ctx_splits;
    } else {
      id = xcd_remap(blockIdx.x - ntree, p.total_groups - ntree);
      rt = id % p.row_tiles;
      id /= p.row_tiles;
      part = id % p.n_ctx_splits;
      id /= p.n_ctx_splits;
    }
  } else {
    id = xcd_remap(blockIdx.x, p.total_groups);
    rt = id % p.row_tiles;
    id /= p.row_tiles;
    part = id % p.n_parts;
    id /= p.n_parts;
  }
  kvh = id % p.Hkv;
  b = id / p.Hkv;
}

#ifndef VA_RING_TILES
#define VA_RING_TILES 2
#endif
template <int RB, int ES, int D, bool GATHER = false>
struct KernelShape {
  // The HBM-bound shapes (bf16, one 32-row block) run one wavefront per SIMD
  // with a ring of register tiles in flight; registers are the larger
  // buffer on a CU (512 KiB vs 160 KiB of LDS).  D = 64 rows are half as
  // long, so a two-tile ring fits as well.
  static constexpr bool hbm_shape = RB == 1 && ES == 2;
  // The gathered (sparse) shape moves few bytes per workgroup and is bound
  // by the latency of its index-then-row loads: two wavefronts per SIMD with
  // one tile each in flight beat one wavefront with a two-tile ring.
  static constexpr bool lat_shape = hbm_shape && GATHER;
  static constexpr int prefetch = lat_shape ? 1 : (hbm_shape ? (D == 128 ? VA_RING_TILES : 2) : 1);
  static constexpr int waves_per_eu = hbm_shape && prefetch == 1 ? 2 : 1;
};

// NT: every K/V row is read by this workgroup only (one row tile per KV
// head), so the loads carry the non-temporal hint.
template <class T, int D, int RB, bool GATHER, bool NT = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(KernelShape<RB, sizeof(T), D, GATHER>::waves_per_eu)))
void partial_kernel(PartialParams p) {
  constexpr int ES = sizeof(T);
  constexpr bool BF = ES == 2;
  constexpr int PF = KernelShape<RB, ES, D, GATHER>::prefetch;
  constexpr int VEC = 16 / ES;                     // elements per 16-byte chunk
  constexpr int CPR = D / VEC;                     // chunks per key row
  constexpr int NCH = kTileKeys * CPR / 64;        // chunks per lane per tile (K or V)
  constexpr int TILE_ELEMS = kTileKeys * D;        // row-major, chunk-swizzled
  constexpr int WAVE_ELEMS = 2 * TILE_ELEMS;       // K tile then V tile
  constexpr int TILES_BYTES = kWaves * WAVE_ELEMS * ES;
  constexpr int QROWS = 32 * RB;
  constexpr int Q_BYTES = BF ? QROWS * D * 2 : 16; // bf16 queries are read from LDS
  constexpr int NDB = D / 32;                      // 32-wide d blocks of O^T
  constexpr int OACC = NDB * RB * 16;              // O^T accumulators per lane
  constexpr int OBUF_BYTES = OACC * 64 * 4;
  constexpr int SMEM_BYTES = TILES_BYTES > OBUF_BYTES ? TILES_BYTES : OBUF_BYTES;
  static_assert(NCH * 64 == kTileKeys * CPR, "tile must split evenly over a wavefront");
  static_assert((CPR & (CPR - 1)) == 0, "chunks per row must be a power of two");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char qsm[Q_BYTES];
  __shared__ uint32_t anc[32 * RB][kAncWords];   // ancestor bits of each row's draft node
  __shared__ int par[kMaxN];
  __shared__ float mbuf[kWaves][RB][32];
  __shared__ float lbuf[RB][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;     // which half of the wavefront
  const int n = lane & 31;     // row (B / C column) owned by this lane

  // ---- which work item
  int rt, part, kvh, b;
  decode_group(p, rt, part, kvh, b);
  if (blockIdx.x == 0 && tid == 0) *p.hdr = p.n_parts;   // for a merge called on its own
  const bool tree = part == p.n_ctx_splits;
  // the last context split of a call whose tree rides on it walks the draft
  // tree after its context keys (dense calls only: no gathered instance)
  const bool tree_after = !GATHER && p.tree_in_last && part == p.n_ctx_splits - 1;
  const int row0 = rt * 32 * RB;

  auto q_row_ptr = [&](int r) __attribute__((always_inline)) -> const T* {
    const int g = r / p.N, i = r % p.N;
    return (const T*)p.q + (int64_t)b * p.qs[0] + (int64_t)(kvh * p.G + g) * p.qs[1] + (int64_t)i * p.qs[2];
  };

  // ---- key range of the walk (this part's context keys, or the draft
  // tree) and its buffer resources
  uint32_t kts_b, vts_b;     // bytes between consecutive keys
  int ke;                    // keys of the walk
  rsrc_t krs, vrs;
  auto set_region = [&](bool tr) __attribute__((always_inline)) {
    const T* kbase;
    const T* vbase;
    int region;              // keys addressable in the region
    if (tr) {
      kbase = (const T*)p.kd + (int64_t)b * p.kds[0] + (int64_t)kvh * p.kds[1];
      vbase = (const T*)p.vd + (int64_t)b * p.vds[0] + (int64_t)kvh * p.vds[1];
      kts_b = (uint32_t)(p.kds[2] * ES);
      vts_b = (uint32_t)(p.vds[2] * ES);
      ke = region = p.N;
    } else {
      kbase = (const T*)p.kc + (int64_t)b * p.kcs[0] + (int64_t)kvh * p.kcs[1];
      vbase = (const T*)p.vc + (int64_t)b * p.vcs[0] + (int64_t)kvh * p.vcs[1];
      kts_b = (uint32_t)(p.kcs[2] * ES);
      vts_b = (uint32_t)(p.vcs[2] * ES);
      ke = p.n_ctx;
      region = p.L;
    }
    krs = make_rsrc(kbase, (uint32_t)region * kts_b);
    vrs = make_rsrc(vbase, (uint32_t)region * vts_b);
  };
  set_region(tree);
  const bool gather = GATHER && !tree;
  const rsrc_t irs = make_rsrc(GATHER ? p.idx + (int64_t)b * p.idx_stride : p.idx, GATHER ? (uint32_t)p.n_ctx * 4u : 0u);
  const int ntiles = ke > 0 ? (ke + kTileKeys - 1) / kTileKeys : 0;
  // Context tiles are dealt out round-robin: at step k the S splits' waves
  // of this (sequence, kv head) read tiles 4(kS + part) + wave, one
  // contiguous window of 4S tiles, which keeps DRAM accesses local.  The
  // tree part walks its (at most 8) tiles with its four waves.
  const int tstep = tree ? kWaves : kWaves * p.n_ctx_splits;
  const int tfirst = tree ? wave : kWaves * part + wave;

  T* kt = (T*)smem + wave * WAVE_ELEMS;
  T* vt = kt + TILE_ELEMS;

  // Chunk c of a lane covers key row kk0 + KPC c of the tile and the
  // 16-byte column col of that row.
  constexpr int KPC = 64 / CPR;
  const int kk0 = lane / CPR;
  const uint32_t col_b = (uint32_t)(lane % CPR) * 16u;

  u32x4 kreg[PF][NCH], vreg[PF][NCH];
  uint32_t vmask[PF];
  int ixr[PF];   // gathered index of key (lane % 32) of the tile each slot loads next

  // Issue the loads of chunk c of tile t into one ring slot.  ix holds the
  // gathered index of key (lane % 32) of the tile (unused when dense).
  auto load_chunk = [&](int t, int c, int ix, u32x4& kr, u32x4& vr) __attribute__((always_inline)) {
    const int key = kTileKeys * t + kk0 + KPC * c;
    uint32_t ko, vo;
    if (GATHER && gather) {
      const int ixc = __shfl(ix, kk0 + KPC * c);
      const bool ok = key < ke && (unsigned)ixc < (unsigned)p.L;
      ko = ok ? (uint32_t)ixc * kts_b + col_b : kOOB;
      vo = ok ? (uint32_t)ixc * vts_b + col_b : kOOB;
    } else {
      ko = (uint32_t)key * kts_b + col_b;   // past the region: reads zeros
      vo = (uint32_t)key * vts_b + col_b;
    }
    kr = buf_load16<NT>(krs, ko);
    vr = buf_load16<NT>(vrs, vo);
  };
  auto load_tile = [&](int t, int ix, u32x4 (&kr)[NCH], u32x4 (&vr)[NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) load_chunk(t, c, ix, kr[c], vr[c]);
  };
  // Keys of tile t that exist (bit j: key 32t + j), from lane n's index.
  auto tile_mask = [&](int t, int ix) __attribute__((always_inline)) -> uint32_t {
    bool ok = kTileKeys * t + n < ke;
    if (GATHER && gather) ok = ok && (unsigned)ix < (unsigned)p.L;
    return (uint32_t)__ballot(ok && h == 0);
  };
  auto load_idx = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (GATHER) return buf_load_i32(irs, (uint32_t)(kTileKeys * t + n) * 4u);
    return 0;
  };

  // ---- fp32 queries stay in registers as MFMA B operands (Q^T)
  constexpr int QREG = BF ? 1 : D / 2;
  float qf[RB][QREG];
  if constexpr (!BF) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row0 + 32 * rb + n;
      const bool ok = r < p.R;
      const T* qrow = q_row_ptr(ok ? r : 0);
#pragma unroll
      for (int ks = 0; ks < QREG; ++ks) qf[rb][ks] = ok ? qrow[2 * ks + h] : 0.f;
    }
  }

  // ---- online softmax state
  float m_run[RB], l_run[RB];
  f32x16 o[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[rb][db][e] = 0.f;
  }
  const float c = p.c;

  // One tile of attention.  MASKED (a compile-time tag) handles tiles with
  // invisible keys (the last context tile, the tree part); whole context
  // tiles take the unmasked instance.  The choice is made before the MFMAs,
  // so no branch separates the S^T chain from the reads of its accumulators.
  auto compute = [&](int t, uint32_t vm, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    uint32_t key_bits[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) key_bits[rb] = MASKED ? vm & anc[32 * rb + n][t & (kAncWords - 1)] : ~0u;

    // S^T = K_tile . Q^T
    f32x16 s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[rb][e] = 0.f;
    if constexpr (BF) {
      const T* qs = (const T*)qsm;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        // keep the scheduler from hoisting every operand read of the tile
        // (register budget of two wavefronts per SIMD)
        if (ks % 2 == 0) __builtin_amdgcn_sched_barrier(0);
        const u32x4 kv = *(const u32x4*)(kt + n * D + swz<CPR>(n, 2 * ks + h) * VEC);
        const bf16x8 a = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int qr = 32 * rb + n;
          const u32x4 qv = *(const u32x4*)(qs + qr * D + swz<CPR>(qr, 2 * ks + h) * VEC);
          s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, qv), s[rb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks) {
        const int d = 2 * ks + h;
        const float a = kt[n * D + swz<CPR>(n, d / VEC) * VEC + d % VEC];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[rb][ks], s[rb], 0, 0, 0);
      }
    }

    // mask, online softmax; s becomes P (unnormalised).  The running max of
    // a row only moves when this tile's max exceeds it by more than 2^8 in
    // exp2 units (lazy rescaling): otherwise P is taken against the stale max
    // (values <= 256, exact enough in fp32 and bf16) and O is left alone.
    // The rescale is one wave-uniform branch, rarely taken after the first
    // tiles.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (MASKED) {
          const int key = 8 * (e >> 2) + 4 * h + (e & 3);
          if (!((key_bits[rb] >> key) & 1u)) s[rb][e] = -INFINITY;
        }
        tmax = fmaxf(tmax, s[rb][e]);
      }
      tmax = half_max(tmax);
      const bool grow = (tmax - m_run[rb]) * c > 8.f;   // false when both are -inf (NaN)
      if (__any(grow)) {
        const float mnew = grow ? tmax : m_run[rb];
        const float alpha = grow ? fast_exp2((m_run[rb] - mnew) * c) : 1.f;
        l_run[rb] *= alpha;
        m_run[rb] = mnew;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[rb][db][e] *= alpha;
      }
      const float mc = m_run[rb] == -INFINITY ? 0.f : m_run[rb] * c;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(s[rb][e], c, -mc));
        s[rb][e] = pe;
        ls += pe;
      }
      l_run[rb] += ls;
    }

    // O^T += V_tile^T . P^T
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (BF) {
      const int bk = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pb[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[rb][j] = (__bf16)s[rb][8 * ks + j];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          __builtin_amdgcn_sched_barrier(0);
          // Transposed LDS reads: this lane receives V[K0 + j][32db + n],
          // j = 0..3, for K0 = 16ks + 4h (k-slots 0..3) and 16ks + 8 + 4h
          // (k-slots 4..7), matching the key order of P^T's k-slots.
          const int d = 32 * db + 16 * (bk & 1) + 4 * (i16 & 3);
          uint32_t w[4];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const int key = 16 * ks + 8 * rr + 4 * h + (i16 >> 2);
            const T* src = vt + key * D + swz<CPR>(key, d >> 3) * VEC + (d & 7);
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const i16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
            const u32x2 tw = __builtin_bit_cast(u32x2, tv);
            w[2 * rr] = tw[0];
            w[2 * rr + 1] = tw[1];
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb], o[rb][db], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + n;
          const float a = vt[key * D + swz<CPR>(key, d / VEC) * VEC + d % VEC];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[rb][e], o[rb][db], 0, 0, 0);
        }
      }
    }
  };

  // ---- stream this wavefront's tiles.  The register copies of the next PF
  // tiles form a ring: each 16-byte chunk is re-issued for the tile PF
  // steps ahead as soon as it has been staged in LDS, so a wavefront keeps
  // about PF tiles of loads in flight at all times.  Loads are never
  // skipped (past the end a slot re-fetches this wavefront's last tile,
  // which is never staged), and the main loop body takes every ring slot
  // with no early exit, so the wait before each staged chunk counts only
  // that slot's older chunks; the last (fewer than PF) tiles are drained
  // after it.
  const int nw = tfirst < ntiles ? (ntiles - 1 - tfirst) / tstep + 1 : 0;   // tiles of this wavefront
  const int klast = nw > 0 ? nw - 1 : 0;
  // A dense context part's last tile may be partial; it is taken last, with
  // the mask.  The other tiles are walked starting at a per-head offset:
  // the K/V regions of all heads lie a power of two apart, and heads walking
  // them in step would crowd the same DRAM channels at the same time.
  const bool partial_last = !tree && !gather && (ke % kTileKeys) != 0 && nw > 0 && tfirst + klast * tstep == ntiles - 1;
  const int nrot = nw - (partial_last ? 1 : 0);
  const int rot = VA_ROTATE && nrot > 0 ? (int)((int64_t)(b * p.Hkv + kvh) * nrot / ((int64_t)p.B * p.Hkv)) : 0;
  auto tile_of = [&](int k) __attribute__((always_inline)) -> int {
    if (k < nrot) {
      const int kr = k + rot;
      return tfirst + (kr >= nrot ? kr - nrot : kr) * tstep;
    }
    return tfirst + (k < klast ? k : klast) * tstep;
  };
#pragma unroll
  for (int pp = 0; pp < PF; ++pp) {
    const int ix = load_idx(tile_of(pp));
    load_tile(tile_of(pp), ix, kreg[pp], vreg[pp]);
    vmask[pp] = tile_mask(tile_of(pp), ix);
    ixr[pp] = load_idx(tile_of(pp + PF));
  }

  // The queries and the tree mask are set up while the ring's first tiles
  // are in flight.
  // ---- bf16 queries of this row tile into LDS (row-major, chunk-swizzled)
  if constexpr (BF) {
    T* qs = (T*)qsm;
    for (int c = tid; c < QROWS * CPR; c += kThreads) {
      const int r = c / CPR, col = c % CPR;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (row0 + r < p.R) v = *(const u32x4*)(q_row_ptr(row0 + r) + col * VEC);
      *(u32x4*)(qs + r * D + swz<CPR>(r, col) * VEC) = v;
    }
  }

  // ---- ancestor bitmasks of the draft tree, one per row of this tile.
  // Ctx parts fill them with ones so the mask lookup needs no branch.
  auto build_anc = [&]() __attribute__((always_inline)) {
    for (int j = tid; j < p.N; j += kThreads) par[j] = p.parent[(int64_t)b * p.N + j];
    for (int j = tid; j < 32 * RB * kAncWords; j += kThreads) (&anc[0][0])[j] = 0u;
    __syncthreads();
    if (tid < 32 * RB && row0 + tid < p.R) {
      int j = (row0 + tid) % p.N;
      for (int step = 0; step <= p.N && j >= 0; ++step) {
        anc[tid][j >> 5] |= 1u << (j & 31);
        int pj = par[j];
        j = (pj >= -1 && pj < j) ? pj : -1;  // malformed parents end the path
      }
    }
    __syncthreads();
  };
  if (tree) {
    build_anc();
  } else {
    for (int j = tid; j < 32 * RB * kAncWords; j += kThreads) (&anc[0][0])[j] = ~0u;
    __syncthreads();
  }

  // Stage ring slot pp in the wavefront's LDS tile; with reload, re-issue
  // each chunk for tile tn right after it is staged.
  auto stage = [&](int pp, bool reload, int tn) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int kk = kk0 + KPC * cc, col = lane % CPR;
      const int off = kk * D + swz<CPR>(kk, col) * VEC;
      *(u32x4*)(kt + off) = kreg[pp][cc];
      *(u32x4*)(vt + off) = vreg[pp][cc];
      if (reload) load_chunk(tn, cc, ixr[pp], kreg[pp][cc], vreg[pp][cc]);
    }
  };
  // Whole ring turns over this wavefront's tiles [0, k_end) with one compute
  // variant; returns the first tile not taken.  The loop body has no early
  // exit and no second compute variant: either would make the compiler
  // drain the ring or duplicate the accumulators across the branches.
  auto ring_loop = [&](int k_end, auto masked_tag) __attribute__((always_inline)) -> int {
    int k = 0;
    for (; k + PF <= k_end; k += PF) {
#pragma unroll
      for (int pp = 0; pp < PF; ++pp) {
        const uint32_t vm = vmask[pp];
        const int tn = tile_of(k + pp + PF);
        stage(pp, true, tn);
        vmask[pp] = tile_mask(tn, ixr[pp]);
        ixr[pp] = load_idx(tile_of(k + pp + 2 * PF));
        compute(tile_of(k + pp), vm, masked_tag);
      }
    }
    return k;
  };
  int k;
  if (!tree && !gather) {
    // dense context: every tile but the part's last is whole (no mask)
    k = ring_loop(nrot, std::false_type{});
  } else {
    // tree and gathered parts run masked: a second (unmasked) variant of
    // the compute step pushes the gathered shape, at two wavefronts per
    // SIMD, past its 256 registers (it spilled and ran ~10% slower)
    k = ring_loop(nw, std::true_type{});
  }
  // the last (at most PF) tiles, already in their ring slots
#pragma unroll
  for (int pp = 0; pp < PF; ++pp) {
    if (k + pp < nw) {
      stage(pp, false, 0);
      compute(tile_of(k + pp), vmask[pp], std::true_type{});
    }
  }
  if constexpr (!GATHER) {
    if (tree_after) {
      // the draft tree's (at most 8) tiles, continuing each wavefront's
      // running softmax: tile t goes to wavefront t mod 4, one at a time
      // through the first ring slot (once every wavefront is done with the
      // all-ones mask of its context tiles)
      __syncthreads();
      build_anc();
      set_region(true);
      for (int t = wave; t < (ke + kTileKeys - 1) / kTileKeys; t += kWaves) {
        load_tile(t, 0, kreg[0], vreg[0]);
        const uint32_t vm = tile_mask(t, 0);
        stage(0, false, 0);
        compute(t, vm, std::true_type{});
      }
    }
  }

  // ---- merge the four wavefronts (fixed order: 3 -> 2 -> 1 -> 0)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] = half_sum(l_run[rb]);
    if (h == 0) mbuf[wave][rb][n] = m_run[rb];
  }
  __syncthreads();
  float m_all[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float M = mbuf[0][rb][n];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mbuf[w][rb][n]);
    m_all[rb] = M;
    const float f = m_run[rb] == -INFINITY ? 0.f : fast_exp2((m_run[rb] - M) * c);
    l_run[rb] *= f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[rb][db][e] *= f;
  }
  float* obuf = (float*)smem;
  for (int w = kWaves - 1; w >= 1; --w) {
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (w != kWaves - 1) l_run[rb] += lbuf[rb][lane];
        lbuf[rb][lane] = l_run[rb];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float* slot = obuf + ((rb * NDB + db) * 16 + e) * 64 + lane;
            if (w != kWaves - 1) o[rb][db][e] += *slot;
            *slot = o[rb][db][e];
          }
      }
    }
    __syncthreads();
  }
  if (wave != 0) return;

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += lbuf[rb][lane];
    const int r = row0 + 32 * rb + n;
    if (r >= p.R) continue;
    const int g = r / p.N, i = r % p.N;
    const int64_t prow = ((int64_t)b * p.Hq + kvh * p.G + g) * p.N + i;
    const float l = l_run[rb];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = p.part_o + (prow * p.part_stride + part) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float acc0 = o[rb][db][4 * q4 + 0] + obuf[((rb * NDB + db) * 16 + 4 * q4 + 0) * 64 + lane];
        const float acc1 = o[rb][db][4 * q4 + 1] + obuf[((rb * NDB + db) * 16 + 4 * q4 + 1) * 64 + lane];
        const float acc2 = o[rb][db][4 * q4 + 2] + obuf[((rb * NDB + db) * 16 + 4 * q4 + 2) * 64 + lane];
        const float acc3 = o[rb][db][4 * q4 + 3] + obuf[((rb * NDB + db) * 16 + 4 * q4 + 3) * 64 + lane];
        float4 v = make_float4(acc0 * inv, acc1 * inv, acc2 * inv, acc3 * inv);
        *(float4*)(dst + 32 * db + 8 * q4 + 4 * h) = v;
      }
    }
    if (h == 0) p.part_lse[prow * p.part_stride + part] = l > 0.f ? m_all[rb] * c + log2f(l) : -INFINITY;
  }
}

// Many query rows per KV head (a large draft tree times the GQA group).
// Eight wavefronts own 32 query rows each (256 rows per workgroup) and share
// every 32-key K/V tile through a three-stage LDS buffer, so K/V bytes are
// read once per 256 rows.  Each wavefront issues the QK MFMAs of the next
// tile before the softmax of the current one, and two wavefronts per SIMD
// let one wavefront's softmax overlap the other's MFMAs.  The workgroup's
// threads keep a ring of RING tiles of 16-byte chunks in flight in
// registers; one LDS barrier per tile.  Every wavefront sees every key of
// the part, so its rows' partials are written directly.
constexpr int kRowsWaves = 8;
constexpr int kRowsThreads = 64 * kRowsWaves;

template <int D, bool GATHER, bool NT = false>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(2)))
void rows_kernel(PartialParams p) {
  using T = uint16_t;
  constexpr int VEC = 8;
  constexpr int CPR = D / VEC;
  constexpr int GROWS = 32 * kRowsWaves;             // rows per workgroup
  // Staged tiles are row-major with padded rows instead of a swizzle, so
  // every LDS read of a lane is one base address plus an immediate offset.
  // K rows (D + 8 elements): the 16 lanes of a 16-byte read cover 64
  // distinct banks.  V rows (D + 32 elements, 16 dwords mod 64 banks): the
  // four keys that a transposed read's lane group touches fall in disjoint
  // bank quarters.
  constexpr int KROW = D + 8;
  constexpr int VROW = D + 32;
  constexpr int TILE_ELEMS = kTileKeys * KROW;       // V tile follows the K tile
  constexpr int STAGE_ELEMS = kTileKeys * (KROW + VROW);
  constexpr int KCH = kTileKeys * CPR;               // chunks of one K (or V) tile
  constexpr int NCT = 2 * KCH / kRowsThreads;        // K+V chunks per thread per tile
  constexpr int NSTAGE = 3;
  constexpr int RING = D == 128 ? 3 : 6;
  constexpr int NDB = D / 32;
  static_assert(NCT >= 1 && NCT * kRowsThreads == 2 * KCH, "tile must split evenly over the workgroup");
  static_assert(RING % NSTAGE == 0, "a whole ring turn keeps LDS buffer indices compile-time");

  __shared__ __attribute__((aligned(16))) T stage[NSTAGE * STAGE_ELEMS];
  __shared__ uint32_t anc[GROWS][kAncWords];
  __shared__ int par[kMaxN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int n = lane & 31;

  int rt, part, kvh, b;
  decode_group(p, rt, part, kvh, b);
  if (blockIdx.x == 0 && tid == 0) *p.hdr = p.n_parts;   // for a merge called on its own
  // tree: a part of the draft tree alone (no context); tree_after: the last
  // context split, which walks the draft tree after its context keys
  const bool tree = part == p.n_ctx_splits;
  const bool tree_after = p.tree_in_last && part == p.n_ctx_splits - 1;
  const int row0 = rt * GROWS;

  // ancestor bitmask of each of the workgroup's rows over the draft nodes
  // (read only by the tree walk; the last context split builds it once its
  // context keys are done, so its context walk starts with the others)
  auto build_anc = [&]() __attribute__((always_inline)) {
    for (int j = tid; j < p.N; j += kRowsThreads) par[j] = p.parent[(int64_t)b * p.N + j];
    for (int j = tid; j < GROWS * kAncWords; j += kRowsThreads) (&anc[0][0])[j] = 0u;
    __syncthreads();
    if (tid < GROWS && row0 + tid < p.R) {
      int j = (row0 + tid) % p.N;
      for (int step = 0; step <= p.N && j >= 0; ++step) {
        anc[tid][j >> 5] |= 1u << (j & 31);
        int pj = par[j];
        j = (pj >= -1 && pj < j) ? pj : -1;  // malformed parents end the path
      }
    }
    __syncthreads();
  };
  if (tree) build_anc();

  // queries of this wavefront's 32 rows as MFMA B operands (Q^T)
  const int myrow = row0 + 32 * wave + n;
  bf16x8 qop[D / 16];
  {
    const bool ok = myrow < p.R;
    const int g = ok ? myrow / p.N : 0, i = ok ? myrow % p.N : 0;
    const T* qrow = (const T*)p.q + (int64_t)b * p.qs[0] + (int64_t)(kvh * p.G + g) * p.qs[1] + (int64_t)i * p.qs[2];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 v = ok ? *(const u32x4*)(qrow + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
      qop[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // the region a walk reads: this split's context keys, or the draft tree
  uint32_t kts_b, vts_b;     // bytes between consecutive keys
  int kb, ke;                // key range of the walk
  rsrc_t krs, vrs;
  bool gather;
  int ntiles, nrot, rot;
  const rsrc_t irs = make_rsrc(GATHER ? p.idx + (int64_t)b * p.idx_stride : p.idx, GATHER ? (uint32_t)p.n_ctx * 4u : 0u);
  auto set_region = [&](bool tr) __attribute__((always_inline)) {
    const T* kbase;
    const T* vbase;
    int region;              // keys addressable in the region
    if (tr) {
      kbase = (const T*)p.kd + (int64_t)b * p.kds[0] + (int64_t)kvh * p.kds[1];
      vbase = (const T*)p.vd + (int64_t)b * p.vds[0] + (int64_t)kvh * p.vds[1];
      kts_b = (uint32_t)(p.kds[2] * 2);
      vts_b = (uint32_t)(p.vds[2] * 2);
      kb = 0;
      ke = region = p.N;
    } else {
      kbase = (const T*)p.kc + (int64_t)b * p.kcs[0] + (int64_t)kvh * p.kcs[1];
      vbase = (const T*)p.vc + (int64_t)b * p.vcs[0] + (int64_t)kvh * p.vcs[1];
      kts_b = (uint32_t)(p.kcs[2] * 2);
      vts_b = (uint32_t)(p.vcs[2] * 2);
      kb = part * p.split_len;
      ke = min(p.n_ctx, kb + p.split_len);
      region = p.L;
    }
    krs = make_rsrc(kbase, (uint32_t)region * kts_b);
    vrs = make_rsrc(vbase, (uint32_t)region * vts_b);
    gather = GATHER && !tr;
    ntiles = ke > kb ? (ke - kb + kTileKeys - 1) / kTileKeys : 0;
    // Tile t of the walk.  Whole context tiles (all but a partial last one)
    // start at a per-head offset, so heads do not read the same DRAM
    // channels in step; the partial tile comes last; past the end a slot
    // re-fetches the last tile, never staged.
    nrot = tr ? 0 : (ke - kb) / kTileKeys;
    rot = VA_ROTATE && nrot > 0 ? (int)((int64_t)(b * p.Hkv + kvh) * nrot / ((int64_t)p.B * p.Hkv)) : 0;
  };
  set_region(tree);

  // Thread chunk j of a tile: combined index tid + 512 j; the first KCH are
  // K chunks, the rest V chunks.  Every chunk of a thread lies in the same
  // key row kk_t of the tile, at 16-byte column col_t.  Whether a chunk is a
  // K or a V chunk depends only on the wavefront.
  const int kk_t = (tid % KCH) / CPR;
  const int col_t = (tid % KCH) % CPR;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  u32x4 rg[RING][NCT];
  bool okr[RING];   // the thread's key exists (tile slot)
  int ixr[RING];    // gathered index of the thread's key in the tile the slot loads next
  auto clamp_tile = [&](int t) __attribute__((always_inline)) -> int {
    if (t < nrot) {
      const int tr = t + rot;
      return tr >= nrot ? tr - nrot : tr;
    }
    return t < ntiles ? t : (ntiles > 0 ? ntiles - 1 : 0);
  };
  auto load_idx = [&](int t) __attribute__((always_inline)) -> int {
    if constexpr (GATHER) return buf_load_i32(irs, (uint32_t)(kb + kTileKeys * clamp_tile(t) + kk_t) * 4u);
    return 0;
  };
  auto load = [&](int t, int ix, u32x4 (&rx)[NCT], bool& ok) __attribute__((always_inline)) {
    const int key = kb + kTileKeys * clamp_tile(t) + kk_t;
    ok = key < ke;
    uint32_t ko = (uint32_t)key * kts_b, vo = (uint32_t)key * vts_b;
    if (GATHER && gather) {
      ok = ok && (unsigned)ix < (unsigned)p.L;
      ko = ok ? (uint32_t)ix * kts_b : kOOB;
      vo = ok ? (uint32_t)ix * vts_b : kOOB;
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const bool isv = 64 * wave_u + kRowsThreads * j >= KCH;
      rx[j] = buf_load16<NT>(isv ? vrs : krs, (isv ? vo : ko) + (uint32_t)col_t * 16u);
    }
  };
  __shared__ int kval[NSTAGE][kTileKeys];   // key of the staged tile exists
  auto stage_write = [&](const u32x4 (&rx)[NCT], bool ok, int buf) __attribute__((always_inline)) {
    T* base = stage + buf * STAGE_ELEMS;
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const bool isv = 64 * wave_u + kRowsThreads * j >= KCH;
      const int off = isv ? TILE_ELEMS + kk_t * VROW + col_t * VEC : kk_t * KROW + col_t * VEC;
      *(u32x4*)(base + off) = rx[j];
    }
    if (tid < KCH && col_t == 0) kval[buf][kk_t] = ok;
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  const float c = p.c;

  // S^T of the tile staged in buffer buf
  auto qk = [&](int buf) __attribute__((always_inline)) -> f32x16 {
    const T* kt = stage + buf * STAGE_ELEMS;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 kv = *(const u32x4*)(kt + n * KROW + (2 * ks + h) * VEC);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv), qop[ks], s, 0, 0, 0);
    }
    return s;
  };
  // online softmax of tile t's scores s, then O^T += V^T P^T
  // mask_tag: 0 no mask (whole context tiles), 1 the tile's existing keys
  // (a partial context tile), 2 existing keys that are ancestors (the tree)
  auto soft_pv = [&](f32x16 s, int t, int buf, auto mask_tag) __attribute__((always_inline)) {
    constexpr int MK = decltype(mask_tag)::value;
    constexpr bool MASKED = MK != 0;
    const T* vt = stage + buf * STAGE_ELEMS + TILE_ELEMS;
    uint32_t key_bits = ~0u;
    if constexpr (MK == 1) key_bits = (uint32_t)__ballot(kval[buf][n] != 0 && h == 0);
    if constexpr (MK == 2)
      key_bits = (uint32_t)__ballot(kval[buf][n] != 0 && h == 0) & anc[32 * wave + n][t & (kAncWords - 1)];

    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (MASKED) {
        const int key = 8 * (e >> 2) + 4 * h + (e & 3);
        if (!((key_bits >> key) & 1u)) s[e] = -INFINITY;
      }
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = half_max(tmax);
    const bool grow = (tmax - m_run) * c > 8.f;
    if (__any(grow)) {
      const float mnew = grow ? tmax : m_run;
      const float alpha = grow ? fast_exp2((m_run - mnew) * c) : 1.f;
      l_run *= alpha;
      m_run = mnew;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    }
    const float mc = m_run == -INFINITY ? 0.f : m_run * c;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = fast_exp2(fmaf(s[e], c, -mc));
      s[e] = pe;
      ls += pe;
    }
    l_run += ls;

    const int bk = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[8 * ks + j];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + 16 * (bk & 1) + 4 * (i16 & 3);
        uint32_t w[4];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int key = 16 * ks + 8 * rr + 4 * h + (i16 >> 2);
          const T* src = vt + key * VROW + d;
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const i16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
          const u32x2 tw = __builtin_bit_cast(u32x2, tv);
          w[2 * rr] = tw[0];
          w[2 * rr + 1] = tw[1];
        }
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]}),
                                                         pb, o[db], 0, 0, 0);
      }
    }
  };
  // Software pipeline over three LDS stages: tiles t and t+1 are staged
  // while tile t is processed, so the QK MFMAs of tile t+1 are issued
  // before the softmax of tile t and run under it; then tile t+2 is staged
  // into the buffer tile t-1 used.
  // prologue of a walk: tiles 0..RING-1 in flight, tiles 0 and 1 staged, S
  // of tile 0
  f32x16 s_cur;
  auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < RING; ++pp) {
      load(pp, load_idx(pp), rg[pp], okr[pp]);
      ixr[pp] = load_idx(pp + RING);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      stage_write(rg[pp], okr[pp], pp);
      load(RING + pp, ixr[pp], rg[pp], okr[pp]);
      ixr[pp] = load_idx(2 * RING + pp);
    }
    lds_barrier();
    s_cur = qk(0);
  };
  prologue();
  auto tile_loop = [&](int t_end, auto masked_tag) __attribute__((always_inline)) {
    int t0 = 0;
    for (; t0 + RING <= t_end; t0 += RING) {
#pragma unroll
      for (int pp = 0; pp < RING; ++pp) {
        const int t = t0 + pp;
        const f32x16 s_nxt = qk((t + 1) % NSTAGE);
        soft_pv(s_cur, t, t % NSTAGE, masked_tag);
        const int nx = (pp + 2) % RING;
        stage_write(rg[nx], okr[nx], (t + 2) % NSTAGE);
        load(t + 2 + RING, ixr[nx], rg[nx], okr[nx]);
        ixr[nx] = load_idx(t + 2 + 2 * RING);
        lds_barrier();
        s_cur = s_nxt;
      }
    }
#pragma unroll
    for (int pp = 0; pp < RING - 1; ++pp) {
      const int t = t0 + pp;
      if (t < t_end) {
        const f32x16 s_nxt = qk((t + 1) % NSTAGE);
        soft_pv(s_cur, t, t % NSTAGE, masked_tag);
        const int nx = (pp + 2) % RING;
        stage_write(rg[nx], okr[nx], (t + 2) % NSTAGE);
        lds_barrier();
        s_cur = s_nxt;
      }
    }
  };
  if (tree) {
    tile_loop(ntiles, std::integral_constant<int, 2>{});
  } else {
    // whole context tiles (dense or gathered) without the mask, then the
    // partial tail tile (staged in buffer nfull % NSTAGE, its S in s_cur)
    // with its existing keys.  A gathered index outside [0, L) in a whole
    // tile reads as a zero key and value row (a precondition violation:
    // memory-safe, result unspecified but finite).
    const int nfull = (ke - kb) / kTileKeys;
    tile_loop(nfull, std::integral_constant<int, 0>{});
    if (nfull < ntiles) soft_pv(s_cur, nfull, nfull % NSTAGE, std::integral_constant<int, 1>{});
    if (tree_after) {
      // the draft tree, continuing this split's running softmax (every
      // wavefront is done with the stages first)
      build_anc();
      set_region(true);
      prologue();
      tile_loop(ntiles, std::integral_constant<int, 2>{});
    }
  }

  // this wavefront's rows: normalised partial and log2-sum-exp
  const float l = half_sum(l_run);
  if (myrow < p.R) {
    const int g = myrow / p.N, i = myrow % p.N;
    const int64_t prow = ((int64_t)b * p.Hq + kvh * p.G + g) * p.N + i;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = p.part_o + (prow * p.part_stride + part) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 v = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                               o[db][4 * q4 + 3] * inv);
        *(float4*)(dst + 32 * db + 8 * q4 + 4 * h) = v;
      }
    if (h == 0) p.part_lse[prow * p.part_stride + part] = l > 0.f ? m_run * c + log2f(l) : -INFINITY;
  }
}

// Output row r of the merge: (sequence, head, node) and the row's parts.
struct MergeRow {
  int i, hq;
  int64_t b;
};
__device__ inline MergeRow merge_row(const MergeParams& p, int64_t prow) {
  // 32-bit division when the row count fits (it always does for real
  // shapes), as it is much cheaper
  MergeRow m;
  if (p.rows <= 0x7fffffff) {
    const uint32_t r32 = (uint32_t)prow, nn = (uint32_t)p.N, hh = (uint32_t)p.Hq;
    const uint32_t bh = r32 / nn;
    m.i = (int)(r32 - bh * nn);
    m.b = bh / hh;
    m.hq = (int)(bh - (uint32_t)m.b * hh);
  } else {
    m.i = (int)(prow % p.N);
    m.hq = (int)((prow / p.N) % p.Hq);
    m.b = prow / ((int64_t)p.N * p.Hq);
  }
  return m;
}

// D / 4 lanes per output row, each holding 16 bytes of every part's row, so
// a wavefront joins 256 / D rows at once; the parts are joined MG at a time.
// A lane loads its row's part log2-sum-exps together with its slices of up to
// MG partial rows (one memory round trip per group, no cross-lane
// reduction); the weights exp2(lse_s - max) then scale the slices.  More than
// MG parts are joined group by group with the running maximum rescaled, as
// in the partial kernels.  The kernel is bound by the round-trip latency of
// its wavefronts, not by bytes: on 32k rows of two parts, two rows per
// wavefront (16-byte loads) took 8.5 us where one row per wavefront (8-byte
// loads, scalar part weights) took 13.7 us; a few thousand rows stay at the
// launch floor either way.
// HDR: the part count is read from the header the partial kernels wrote
// (a merge called on its own after a shape whose dense and sparse plans
// join different part counts), kept inside the workspace's slots.
template <class T, int D, int MG, bool HDR>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int PER = 4;                 // values per lane: 16 bytes of each part's row
  constexpr int LPR = D / PER;           // lanes per row
  constexpr int RPW = 64 / LPR;          // rows per wavefront
  const int lane = threadIdx.x & 63;
  const int64_t prow = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  // no lane of the wavefront talks to another, so a lane past the last row
  // simply leaves
  if (prow >= p.rows) return;
  const float* lse2 = p.part_lse + prow * p.part_stride;
  const float* po = p.part_o + prow * p.part_stride * D + (lane % LPR) * PER;

  float m_run = -INFINITY, wsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  // part slot s of this row into (lv, v)
  auto load_slot = [&](int s, float& lv, float (&v)[PER]) __attribute__((always_inline)) {
    lv = lse2[s];
    const float4 t = *(const float4*)(po + (int64_t)s * D);
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
  };
  // join the first cnt of G loaded parts into the running (m_run, wsum, acc)
  auto join = [&](auto g_tag, int cnt, bool first, const float* lv, const float (*v)[PER]) __attribute__((always_inline)) {
    constexpr int G = decltype(g_tag)::value;
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (u < cnt) gm = fmaxf(gm, lv[u]);
    const float mnew = fmaxf(m_run, gm);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    if (!first) {
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - muse);
      wsum *= alpha;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (u < cnt) {
        const float w = exp2f(lv[u] - muse);
        wsum += w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
    m_run = mnew;
  };
  if constexpr (HDR) {
    // The part count comes from the header the partial kernels wrote (kept
    // inside the workspace's slots).  The slots are loaded before it is
    // known, with indices clamped to the last slot, in groups of 8 (a slot
    // past the part count is loaded but not used), so the header's latency
    // overlaps the loads.
    constexpr int GH = 8;
    const int hv = *p.hdr;
    const int last = p.part_stride - 1;
    float lv[GH], v[GH][PER];
#pragma unroll
    for (int u = 0; u < GH; ++u) load_slot(min(u, last), lv[u], v[u]);
    __builtin_amdgcn_sched_barrier(0);   // the header's first use after the loads
    const int np = min(max(hv, 1), p.part_stride);
    join(std::integral_constant<int, GH>{}, min(GH, np), true, lv, v);
    for (int s0 = GH; s0 < np; s0 += GH) {
#pragma unroll
      for (int u = 0; u < GH; ++u) load_slot(min(s0 + u, last), lv[u], v[u]);
      join(std::integral_constant<int, GH>{}, min(GH, np - s0), false, lv, v);
    }
  } else {
    const int np = p.n_parts;
    for (int s0 = 0; s0 < np; s0 += MG) {
      const int cnt = min(MG, np - s0);
      float lv[MG], v[MG][PER];
#pragma unroll
      for (int u = 0; u < MG; ++u) {
        lv[u] = -INFINITY;
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = 0.f;
        if (u < cnt) load_slot(s0 + u, lv[u], v[u]);   // uniform: only the parts that exist
      }
      join(std::integral_constant<int, MG>{}, cnt, s0 == 0, lv, v);
    }
  }
  const MergeRow mr = merge_row(p, prow);
  const float muse = m_run == -INFINITY ? 0.f : m_run;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* orow = (T*)p.out + mr.b * p.os[0] + (int64_t)mr.hq * p.os[1] + (int64_t)mr.i * p.os[2] + (lane % LPR) * PER;
  if constexpr (sizeof(T) == 2) {
    uint32_t h[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[e] * inv));
    *(uint2*)orow = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  } else {
    *(float4*)orow = float4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  }
  if (p.lse != nullptr && lane % LPR == 0)
    p.lse[prow] = wsum > 0.f ? (muse + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
}

template <class T, int D, int RB, bool G, bool NT = false>
hipError_t launch_p(const PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((partial_kernel<T, D, RB, G, NT>), dim3(p.total_groups), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// The non-temporal hint goes on dense bf16 reads with one row tile per KV
// head (each K/V row read once), of 32 or 64 rows; with several row tiles
// the later tiles find the rows in L2.
template <class T, int D>
hipError_t launch_p_rb(const PartialParams& p, int rb, bool gather, hipStream_t stream) {
  const bool nt = sizeof(T) == 2 && !gather && p.row_tiles == 1;
  if (rb == 1) {
    if (gather) return launch_p<T, D, 1, true>(p, stream);
    if (nt) return launch_p<T, D, 1, false, true>(p, stream);
    return launch_p<T, D, 1, false>(p, stream);
  }
  if (gather) return launch_p<T, D, 2, true>(p, stream);
  if (nt) return launch_p<T, D, 2, false, true>(p, stream);
  return launch_p<T, D, 2, false>(p, stream);
}

template <int D, bool G>
hipError_t launch_rows(const PartialParams& p, hipStream_t stream) {
  if (!G && p.row_tiles == 1)
    hipLaunchKernelGGL((rows_kernel<D, G, true>), dim3(p.total_groups), dim3(kRowsThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((rows_kernel<D, G>), dim3(p.total_groups), dim3(kRowsThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partials(const PartialParams& p, int dtype, int D, int rb, bool gather,
                           hipStream_t stream) {
  if (rb == kRowsKernel) {
    if (D == 64) return gather ? launch_rows<64, true>(p, stream) : launch_rows<64, false>(p, stream);
    return gather ? launch_rows<128, true>(p, stream) : launch_rows<128, false>(p, stream);
  }
  if (dtype == 1) {
    return D == 64 ? launch_p_rb<uint16_t, 64>(p, rb, gather, stream)
                   : launch_p_rb<uint16_t, 128>(p, rb, gather, stream);
  }
  return D == 64 ? launch_p_rb<float, 64>(p, rb, gather, stream)
                 : launch_p_rb<float, 128>(p, rb, gather, stream);
}

template <class T, int D>
void launch_merge_d(const MergeParams& p, hipStream_t stream) {
  constexpr int rows_per_group = 4 * (256 / D);   // four wavefronts of 64 / (D / 4) rows
  const dim3 grid((unsigned)((p.rows + rows_per_group - 1) / rows_per_group));
  if (p.n_parts == 0)
    hipLaunchKernelGGL((merge_kernel<T, D, 8, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((merge_kernel<T, D, 8, false>), grid, dim3(256), 0, stream, p);
}

hipError_t launch_merge(const MergeParams& p, int dtype, int D, hipStream_t stream) {
  if (dtype == 1) {
    if (D == 64)
      launch_merge_d<uint16_t, 64>(p, stream);
    else
      launch_merge_d<uint16_t, 128>(p, stream);
  } else {
    if (D == 64)
      launch_merge_d<float, 64>(p, stream);
    else
      launch_merge_d<float, 128>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace va
