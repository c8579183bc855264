// Internal declarations shared by the host API and the kernels of
// libverify_attn.so.  Not installed; the public interface is verify_attn.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace va {

// How one verification call is cut into workgroups.
//
// Rows: the G * N query rows that share one KV head (G query heads of the
// group times N draft nodes) are cut into row tiles of 32 * rb rows.
// Keys: the n_ctx context keys are cut into n_ctx_splits splits of
// split_len keys; the draft (tree) keys form one more part.  Every
// (sequence, kv head, row tile, part) is one workgroup that writes one
// normalised partial output and its log2-sum-exp.  The plan of a dense call
// can differ from that of a sparse call of the same shape and n_ctx; the
// workspace layout cannot (it holds part_stride partial slots per row, the
// larger of the two part counts, and a header with the part count the
// partial kernels used).
// Plan::rb value selecting rows_kernel (bf16, many query rows per KV head:
// 256 rows per workgroup, 32 per wavefront, K/V tiles shared in LDS).
constexpr int kRowsKernel = 8;

struct Plan {
  int rb;            // 32-row blocks per wave (1 or 2), or kRowsKernel
  int row_tiles;     // ceil(G * N / (32 * rb))
  int split_len;     // context keys per split (multiple of 128)
  int n_ctx_splits;  // ceil(n_ctx / split_len); 0 when n_ctx == 0
  int n_parts;       // n_ctx_splits + 1 (the tree part is last), or n_ctx_splits when tree_in_last
  int tree_in_last;  // the shared-tile kernel's last split also walks the draft tree
  int part_stride;   // partial slots per row in the workspace (either mode's n_parts fits)
  int64_t rows;      // B * Hq * N output rows
  size_t off_lse;    // byte offset of the partial lse array in the workspace
  size_t off_hdr;    // byte offset of the header (int32 n_parts written by the partial kernels)
  size_t ws_bytes;   // total workspace bytes
};

struct PartialParams {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kd;
  const void* vd;
  const int32_t* parent;
  const int32_t* idx;   // verify set (sparse) or nullptr (dense)
  int64_t idx_stride;
  int64_t qs[3], kcs[3], vcs[3], kds[3], vds[3];
  float* part_o;        // [rows][part_stride][D], slots [0, n_parts) written
  float* part_lse;      // [rows][part_stride], log2 domain
  int* hdr;             // workspace header: n_parts, written by workgroup 0
  int B, Hq, Hkv, G, N, L, n_ctx;
  int R;                // G * N
  int row_tiles, split_len, n_ctx_splits, n_parts, part_stride;
  int tree_in_last;     // no tree part: the last context split walks the tree too
  int total_groups;     // grid size
  float c;              // scale * log2(e)
};

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;           // may be nullptr
  int64_t os[3];
  int64_t rows;
  int Hq, N;
  int n_parts;          // parts to join, or 0: read them from hdr (clamped to [1, part_stride])
  int part_stride;      // partial slots per row
  const int* hdr;       // workspace header written by the partial kernels
};

struct CommitParams {
  void* kc;
  void* vc;
  const void* kd;
  const void* vd;
  const int32_t* parent;
  const int32_t* accepted;
  const int32_t* cache_len;
  int32_t* new_len;
  int64_t kcs[3], vcs[3], kds[3], vds[3];
  int B, Hkv, N, capacity, es, row_bytes;
};

struct ScoreParams {
  const void* q;        // [B, Hs, M, D] bf16 (strides qs)
  const void* k;        // [B, Hs, L, D] bf16 (strides ks)
  int64_t qs[3], ks[3];
  float* score;         // [B, L] fp32, row stride ld_out
  int64_t ld_out;
  float* s;             // workspace: scaled scores [B, Hs, M, ld_s], log2 domain
  float* stat_m;        // workspace: [B, Hs, M, n_splits] split max
  float* stat_l;        // workspace: [B, Hs, M, n_splits] split sum
  int64_t ld_s;         // L rounded up to 32
  int B, Hs, M, L;
  int split_len, n_splits, total_groups;
  float c;              // scale * log2(e)
};

constexpr int kTreeMaxKT = 4096;   // K * T candidates per sequence
constexpr int kTreeMaxN = 256;

struct TreeParams {
  const float* prob;      // [B, K, T]
  const int32_t* tok;     // [B, K, T]
  int32_t* parent;        // [B, N]
  int32_t* token;         // [B, N]
  float* rho;             // [B, N]
  float* a_hat;           // [B]
  int B, K, T, N;
};

// Launchers (va_attn.hip, va_commit.hip, va_score.hip, va_tree.hip).  Return
// the hipError_t of the launch.
hipError_t launch_tree(const TreeParams& p, hipStream_t stream);
hipError_t launch_scores(const ScoreParams& p, int D, hipStream_t stream);
hipError_t launch_recovery(const float* score, int64_t ld, int B, int L, const int32_t* idx, int K,
                           int64_t idx_stride, int rows, int accumulate, float* arr, hipStream_t stream);
hipError_t launch_commit(const CommitParams& p, hipStream_t stream);
hipError_t launch_partials(const PartialParams& p, int dtype, int D, int rb, bool gather,
                           hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int dtype, int D, hipStream_t stream);

}  // namespace va
