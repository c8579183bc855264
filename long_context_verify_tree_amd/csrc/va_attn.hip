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
//                   part S is the draft tree under its ancestor mask.
//                   Writes a normalised partial row and its log2-sum-exp.
//   merge_kernel    one wavefront per output row: log-sum-exp merge of the
//                   S + 1 partials with wavefront shuffles.
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

#include <hip/hip_runtime.h>

#include "va_internal.h"

namespace va {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte vector used for every global/LDS move.  may_alias: LDS tiles are
// written through this type and read back as bf16 / float elements.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), __may_alias__));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 32;
constexpr int kMaxN = 256;
constexpr int kAncWords = kMaxN / 32;

__device__ inline int xcd_remap(int x, int total) {
  // Workgroups are dispatched round-robin over the 8 XCDs (x % 8).  Give each
  // XCD a contiguous range of logical ids so neighbours (row tiles of one
  // split) share that XCD's L2.
  const int q = total / 8, r = total % 8;
  const int xcd = x % 8, local = x / 8;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two wavefronts per SIMD where the registers allow it (one 32-row block):
// twice the K/V bytes in flight per CU for the HBM-bound shapes.
template <class T, int D, int RB, bool GATHER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RB == 1 && sizeof(T) == 2 ? 2 : 1)))
void partial_kernel(PartialParams p) {
  constexpr int ES = sizeof(T);
  constexpr int VEC = 16 / ES;                     // elements per 16-byte chunk
  constexpr int LDR = D + VEC;                     // LDS row stride (elements), 16 B pad
  constexpr int CPR = D / VEC;                     // chunks per key row
  constexpr int NCH = kTileKeys * CPR / 64;        // chunks per lane per tile (K or V)
  constexpr int TILE_ELEMS = kTileKeys * LDR;      // K tile, key-major rows
  // V tile stored transposed (d-major rows of the tile's 32 keys) so an MFMA
  // A operand of V^T is two 8-byte reads.  Row stride padded to spread banks.
  constexpr int VT_LDR = (ES == 2) ? kTileKeys + 4 : kTileKeys + 1;
  constexpr int VT_ELEMS = D * VT_LDR;
  constexpr int WAVE_ELEMS = TILE_ELEMS + VT_ELEMS;  // K tile then V^T tile
  constexpr int TILES_BYTES = kWaves * WAVE_ELEMS * ES;
  constexpr int NDB = D / 32;                      // 32-wide d blocks of O^T
  constexpr int OACC = NDB * RB * 16;              // O^T accumulators per lane
  constexpr int OBUF_BYTES = OACC * 64 * 4;
  constexpr int SMEM_BYTES = TILES_BYTES > OBUF_BYTES ? TILES_BYTES : OBUF_BYTES;
  static_assert(NCH * 64 == kTileKeys * CPR, "tile must split evenly over a wavefront");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
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
  int id = xcd_remap(blockIdx.x, p.total_groups);
  const int rt = id % p.row_tiles;
  id /= p.row_tiles;
  const int part = id % p.n_parts;
  id /= p.n_parts;
  const int kvh = id % p.Hkv;
  const int b = id / p.Hkv;
  const bool tree = part == p.n_ctx_splits;
  const int row0 = rt * 32 * RB;

  // ---- ancestor bitmasks of the draft tree, one per row of this tile.
  // Ctx parts fill them with ones so the mask lookup needs no branch.
  if (tree) {
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
  } else {
    for (int j = tid; j < 32 * RB * kAncWords; j += kThreads) (&anc[0][0])[j] = ~0u;
    __syncthreads();
  }

  // ---- queries of this lane's rows as MFMA B operands (Q^T)
  constexpr int QOPS = (ES == 2) ? D / 16 : D / 2;
  typedef typename std::conditional<ES == 2, bf16x8, float>::type QOp;
  QOp qop[RB][QOPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + 32 * rb + n;
    const bool ok = r < p.R;
    const int g = ok ? r / p.N : 0;
    const int i = ok ? r % p.N : 0;
    const T* qrow = (const T*)p.q + (int64_t)b * p.qs[0] + (int64_t)(kvh * p.G + g) * p.qs[1] +
                    (int64_t)i * p.qs[2];
#pragma unroll
    for (int ks = 0; ks < QOPS; ++ks) {
      if constexpr (ES == 2) {
        u32x4 v = ok ? *(const u32x4*)(qrow + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
        qop[rb][ks] = __builtin_bit_cast(bf16x8, v);
      } else {
        qop[rb][ks] = ok ? qrow[2 * ks + h] : 0.f;
      }
    }
  }

  // ---- key range of this part
  const T* kbase;
  const T* vbase;
  int64_t kts, vts;
  int kb, ke;
  if (tree) {
    kbase = (const T*)p.kd + (int64_t)b * p.kds[0] + (int64_t)kvh * p.kds[1];
    vbase = (const T*)p.vd + (int64_t)b * p.vds[0] + (int64_t)kvh * p.vds[1];
    kts = p.kds[2];
    vts = p.vds[2];
    kb = 0;
    ke = p.N;
  } else {
    kbase = (const T*)p.kc + (int64_t)b * p.kcs[0] + (int64_t)kvh * p.kcs[1];
    vbase = (const T*)p.vc + (int64_t)b * p.vcs[0] + (int64_t)kvh * p.vcs[1];
    kts = p.kcs[2];
    vts = p.vcs[2];
    kb = part * p.split_len;
    ke = min(p.n_ctx, kb + p.split_len);
  }
  const bool gather = GATHER && !tree;
  const int32_t* idx_row = GATHER ? p.idx + (int64_t)b * p.idx_stride : nullptr;
  const int ntiles = ke > kb ? (ke - kb + kTileKeys - 1) / kTileKeys : 0;

  T* kt = (T*)smem + wave * WAVE_ELEMS;
  T* vt = kt + TILE_ELEMS;   // V^T: vt[d * VT_LDR + key]

  u32x4 kreg[NCH], vreg[NCH];
  uint32_t vmask_next = 0;

  auto key_pos = [&](int key, bool& ok) -> int64_t {
    ok = key < ke;
    if (gather && ok) {
      const int ix = idx_row[key];
      ok = (unsigned)ix < (unsigned)p.L;
      return ix;
    }
    return key;
  };

  auto load_tile = [&](int t) {
    const int key0 = kb + kTileKeys * t;
    // K: chunk c of lane -> (key kk, column col): 16-byte pieces of whole rows.
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int chunk = lane + 64 * c;
      const int kk = chunk / CPR, col = chunk % CPR;
      bool ok;
      const int64_t pos = key_pos(key0 + kk, ok);
      kreg[c] = ok ? *(const u32x4*)(kbase + pos * kts + col * VEC) : u32x4{0, 0, 0, 0};
    }
    // V: lane -> key (lane % 32), columns 2c + lane / 32, so the transposed
    // LDS writes of one instruction cover consecutive keys of one d row.
    bool vok;
    const int64_t vpos = key_pos(key0 + n, vok);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = 2 * c + h;
      vreg[c] = vok ? *(const u32x4*)(vbase + vpos * vts + col * VEC) : u32x4{0, 0, 0, 0};
    }
    vmask_next = (uint32_t)__ballot(vok && h == 0);
  };

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

  int t = wave;
  if (t < ntiles) load_tile(t);
  for (; t < ntiles; t += kWaves) {
    // stage the fetched tile in this wavefront's LDS tile
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int chunk = lane + 64 * cc;
      const int kk = chunk / CPR, col = chunk % CPR;
      *(u32x4*)(kt + kk * LDR + col * VEC) = kreg[cc];
      // V^T: the VEC elements of this chunk go to rows d = (2cc + h) * VEC + e
      const int d0 = (2 * cc + h) * VEC;
      if constexpr (ES == 2) {
        const uint32_t w[4] = {vreg[cc][0], vreg[cc][1], vreg[cc][2], vreg[cc][3]};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vt[(d0 + e) * VT_LDR + n] = (T)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (element copied to a scalar first: bit-casting a vector-element
          // subscript directly yields element 0 with this compiler)
          const uint32_t x = vreg[cc][e];
          vt[(d0 + e) * VT_LDR + n] = __uint_as_float(x);
        }
      }
    }
    const uint32_t vmask = vmask_next;
    if (t + kWaves < ntiles) load_tile(t + kWaves);  // in flight during the math below

    // Visible keys of this tile per row, computed before the MFMAs so that no
    // branch separates the S^T chain from the reads of its accumulators.
    uint32_t key_bits[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) key_bits[rb] = vmask & anc[32 * rb + n][t & (kAncWords - 1)];

    // S^T = K_tile . Q^T
    f32x16 s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[rb][e] = 0.f;
    if constexpr (ES == 2) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kv = *(const u32x4*)(kt + n * LDR + 16 * ks + 8 * h);
        const bf16x8 a = __builtin_bit_cast(bf16x8, kv);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[rb][ks], s[rb], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks) {
        const float a = kt[n * LDR + 2 * ks + h];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[rb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qop[rb][ks], s[rb], 0, 0, 0);
      }
    }

    // mask, online softmax; s becomes P (unnormalised)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t bits = key_bits[rb];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * h + (e & 3);
        if (!((bits >> key) & 1u)) s[rb][e] = -INFINITY;
        tmax = fmaxf(tmax, s[rb][e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(m_run[rb], tmax);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = fast_exp2((m_run[rb] - muse) * c);
      const float mc = muse * c;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(s[rb][e], c, -mc));
        s[rb][e] = pe;
        ls += pe;
      }
      l_run[rb] = l_run[rb] * alpha + ls;
      m_run[rb] = mnew;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[rb][db][e] *= alpha;
    }

    // O^T += V_tile^T . P^T
    if constexpr (ES == 2) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pb[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[rb][j] = (__bf16)s[rb][8 * ks + j];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // k-slots j = 0..3: keys 16ks + 4h + j; j = 4..7: keys 16ks + 8 + 4h + (j - 4)
          const T* vrow = vt + (32 * db + n) * VT_LDR + 16 * ks + 4 * h;
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2), __may_alias__));
          const u32x2 lo = *(const u32x2*)(vrow);
          const u32x2 hi = *(const u32x2*)(vrow + 8);
          const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
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
          const float a = vt[(32 * db + n) * VT_LDR + key];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[rb][e], o[rb][db], 0, 0, 0);
        }
      }
    }
  }

  // ---- merge the four wavefronts (fixed order: 3 -> 2 -> 1 -> 0)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] += __shfl_xor(l_run[rb], 32);
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
    float* dst = p.part_o + (prow * p.n_parts + part) * D;
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
    if (h == 0) p.part_lse[prow * p.n_parts + part] = l > 0.f ? m_all[rb] * c + log2f(l) : -INFINITY;
  }
}

template <class T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  // One wavefront per output row.  Lane s holds part s's log2-sum-exp; the
  // maximum and the weight sum are wavefront shuffle reductions; the weights
  // are broadcast with readlane, so the partial-row loads are independent of
  // one another and stay in flight together.
  const int lane = threadIdx.x & 63;
  const int64_t prow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (prow >= p.rows) return;
  const int i = (int)(prow % p.N);
  const int hq = (int)((prow / p.N) % p.Hq);
  const int64_t b = prow / ((int64_t)p.N * p.Hq);
  const float* lse2 = p.part_lse + prow * p.n_parts;
  const int np = p.n_parts;

  float M = -INFINITY;
  for (int s = lane; s < np; s += 64) M = fmaxf(M, lse2[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float muse = M == -INFINITY ? 0.f : M;

  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  const float* po = p.part_o + prow * np * D + lane * PER;
  for (int s0 = 0; s0 < np; s0 += 64) {
    const int cnt = min(64, np - s0);
    const float wl = lane < cnt ? exp2f(lse2[s0 + lane] - muse) : 0.f;
    float ws = wl;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
    wsum += ws;
    int s = 0;
    for (; s + 8 <= cnt; s += 8) {
      float v[8][PER];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = po[(int64_t)(s0 + s + u) * D + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s + u));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, v[u][e], acc[e]);
      }
    }
    for (; s < cnt; ++s) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, po[(int64_t)(s0 + s) * D + e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* orow = (T*)p.out + b * p.os[0] + (int64_t)hq * p.os[1] + (int64_t)i * p.os[2] + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float v = acc[e] * inv;
    if constexpr (sizeof(T) == 2) {
      orow[e] = __builtin_bit_cast(uint16_t, (__bf16)v);
    } else {
      orow[e] = v;
    }
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[prow] = wsum > 0.f ? (muse + log2f(wsum)) * 0.69314718055994530942f : -INFINITY;
}

template <class T, int D, int RB, bool G>
hipError_t launch_p(const PartialParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((partial_kernel<T, D, RB, G>), dim3(p.total_groups), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class T, int D>
hipError_t launch_p_rb(const PartialParams& p, int rb, bool gather, hipStream_t stream) {
  if (rb == 1) return gather ? launch_p<T, D, 1, true>(p, stream) : launch_p<T, D, 1, false>(p, stream);
  return gather ? launch_p<T, D, 2, true>(p, stream) : launch_p<T, D, 2, false>(p, stream);
}

}  // namespace

hipError_t launch_partials(const PartialParams& p, int dtype, int D, int rb, bool gather,
                           hipStream_t stream) {
  if (dtype == 1) {
    return D == 64 ? launch_p_rb<uint16_t, 64>(p, rb, gather, stream)
                   : launch_p_rb<uint16_t, 128>(p, rb, gather, stream);
  }
  return D == 64 ? launch_p_rb<float, 64>(p, rb, gather, stream)
                 : launch_p_rb<float, 128>(p, rb, gather, stream);
}

hipError_t launch_merge(const MergeParams& p, int dtype, int D, hipStream_t stream) {
  const unsigned grid = (unsigned)((p.rows + 3) / 4);
  if (dtype == 1) {
    if (D == 64)
      hipLaunchKernelGGL((merge_kernel<uint16_t, 64>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<uint16_t, 128>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((merge_kernel<float, 64>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<float, 128>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace va
