// Host side of libverify_attn.so: argument validation, work planning and
// kernel launches behind the C ABI of include/verify_attn.h.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing.  The library keeps no state between calls.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/verify_attn.h"
#include "va_internal.h"
#include "va_select.h"

namespace {

thread_local char g_msg[512] = "";

va_status fail(va_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

va_status ok() {
  g_msg[0] = '\0';
  return VA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

va_status check_desc(const va_attn_desc* d) {
  if (d == nullptr) return fail(VA_EINVAL, "desc is NULL");
  if (d->B < 1 || d->Hq < 1 || d->Hkv < 1) return fail(VA_EINVAL, "B, Hq, Hkv must be >= 1");
  if (d->Hq % d->Hkv != 0) return fail(VA_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", d->Hq, d->Hkv);
  if (d->L < 0) return fail(VA_EINVAL, "L must be >= 0");
  if (d->N < 1) return fail(VA_EINVAL, "N must be >= 1");
  if (d->N > 256) return fail(VA_EUNSUPPORTED, "N = %d exceeds 256 draft nodes", d->N);
  if (d->D != 64 && d->D != 128) return fail(VA_EUNSUPPORTED, "D = %d (supported: 64, 128)", d->D);
  if (d->dtype != VA_FP32 && d->dtype != VA_BF16) return fail(VA_EINVAL, "unknown dtype %d", d->dtype);
  if (isnan(d->scale) || isinf(d->scale)) return fail(VA_EINVAL, "scale must be finite");
  const int64_t vec = d->dtype == VA_BF16 ? 8 : 4;  // elements per 16 bytes
  const int64_t* strides[6] = {d->q_stride, d->kc_stride, d->vc_stride, d->kd_stride, d->vd_stride, d->o_stride};
  const char* names[6] = {"q", "k_cache", "v_cache", "k_draft", "v_draft", "out"};
  for (int t = 0; t < 6; ++t)
    for (int a = 0; a < 3; ++a)
      if (strides[t][a] % vec != 0)
        return fail(VA_EINVAL, "%s stride[%d] = %lld breaks 16-byte row alignment", names[t], a,
                    (long long)strides[t][a]);
  // The kernels address the keys of one (sequence, kv head) with 32-bit byte
  // offsets from that region's start: positive key strides, region (plus a
  // margin of 64 keys) under 2^31 bytes.
  const int64_t es = d->dtype == VA_BF16 ? 2 : 4;
  for (int t = 1; t <= 4; ++t) {
    const int64_t keys = (t <= 2 ? (int64_t)d->L : (int64_t)d->N) + 64;
    if (strides[t][2] <= 0)
      return fail(VA_EUNSUPPORTED, "%s key stride must be positive (got %lld)", names[t], (long long)strides[t][2]);
    if (keys * strides[t][2] * es > ((int64_t)1 << 31))
      return fail(VA_EUNSUPPORTED, "%s: %lld keys x %lld-byte stride exceed the 2 GiB per-head region limit",
                  names[t], (long long)keys - 64, (long long)(strides[t][2] * es));
  }
  return VA_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// Byte ranges [a, a + na) and [b, b + nb) share an address.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// The work cut of one call (kernel, row tiles, splits, parts), which
// depends on whether the call is dense or sparse.
va::Plan plan_cut(const va_attn_desc* d, int32_t n_ctx, bool sparse) {
  va::Plan pl{};
  const int G = d->Hq / d->Hkv;
  const int R = G * d->N;
  // bf16 with more than 64 query rows per KV head: the shared-tile rows
  // kernel (256 rows per workgroup).  bf16 with 33 to 64 rows: in a dense
  // call one 64-row tile (two row blocks per wavefront, one wavefront per
  // SIMD), so each streamed K/V row feeds 64 rows in one workgroup; in a
  // sparse call two 32-row tiles, as the gathered rows are bound by load
  // latency and the 64-row tile keeps half as many wavefronts loading.
  // Other bf16 shapes: 32-row tiles.  fp32: 32 or 64 rows.
#ifndef VA_ROWS_MIN_R
#define VA_ROWS_MIN_R 64
#endif
  if (d->dtype == VA_BF16)
    pl.rb = R > VA_ROWS_MIN_R ? va::kRowsKernel : (R > 32 && !sparse ? 2 : 1);
  else
    pl.rb = R <= 32 ? 1 : 2;
  const int rows_per_tile = pl.rb == va::kRowsKernel ? 256 : 32 * pl.rb;
  pl.row_tiles = (R + rows_per_tile - 1) / rows_per_tile;
  const int64_t pairs = (int64_t)d->B * d->Hkv * pl.row_tiles;
  // Context splits.  The partial kernels run about one workgroup per CU,
  // so the context workgroups run in rounds of 256, each round as long as
  // its splits.  Of the split counts up to twice the one that first reaches
  // 256 workgroups, take the one whose rounds finish first (rounds x keys
  // per split, after rounding a split to a multiple of 128 keys and at least
  // 512), the fewest splits on a tie: every split costs one partial row per
  // query row in the workspace.  (Reaching 256 workgroups alone can leave a
  // few in a second round on an idle chip: 96 pairs in 3 splits are 288
  // workgroups, two rounds of a third of the context; 5 splits take two
  // rounds of a fifth.)
#ifndef VA_TARGET_GROUPS
#define VA_TARGET_GROUPS 256
#endif
#ifndef VA_MIN_SPLIT
#define VA_MIN_SPLIT 512
#endif
  const int64_t target_groups = VA_TARGET_GROUPS;
  const int64_t s0 = pairs < target_groups ? (target_groups + pairs - 1) / pairs : 1;
  int64_t best_len = VA_MIN_SPLIT, best_splits = 0, best_cost = -1;
  // from ceil(n_ctx / min split) on, every count makes the same minimum-length
  // splits: the search stops there (the choice is unchanged)
  const int64_t s_cap = (n_ctx + VA_MIN_SPLIT - 1) / VA_MIN_SPLIT;
  const int64_t s_end = 2 * s0 < s_cap ? 2 * s0 : s_cap;
  for (int64_t s = 1; s <= s_end && n_ctx > 0; ++s) {
    int64_t len = (n_ctx + s - 1) / s;
    len = (len + 127) / 128 * 128;
    if (len < VA_MIN_SPLIT) len = VA_MIN_SPLIT;
    const int64_t splits = (n_ctx + len - 1) / len;
    const int64_t cost = (pairs * splits + target_groups - 1) / target_groups * len;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_len = len;
      best_splits = splits;
    }
  }
  pl.split_len = (int)best_len;
  pl.n_ctx_splits = (int)best_splits;
  // The shared-tile kernel runs one workgroup per CU: the tree rides on the
  // last context split's workgroup (after its context keys), so the grid is
  // the context workgroups alone and each row has one partial row fewer.
  // The per-wavefront kernels do the same in a dense call whose context
  // workgroups fill the chip (otherwise a tree workgroup of its own runs
  // beside them on an idle CU); in a sparse call they keep the tree as a
  // part of its own (short workgroups that start first): the gathered
  // kernel runs two workgroups per CU, so its tree workgroups displace no
  // context workgroup.
  const bool fills = pairs * pl.n_ctx_splits >= target_groups;
  pl.tree_in_last = pl.n_ctx_splits > 0 && (pl.rb == va::kRowsKernel || (!sparse && fills));
  // The shared-tile kernel walks each split as one contiguous key range, so
  // when its last split also walks the N tree keys, the other splits take
  // those keys' worth more context: every split then walks about
  // (n_ctx + N) / S keys (rounded up to whole 32-key tiles), and none more
  // than before.  (The per-wavefront kernel deals its tiles round-robin
  // over the splits.)
  if (pl.tree_in_last && pl.rb == va::kRowsKernel && pl.n_ctx_splits > 1) {
    const int64_t S = pl.n_ctx_splits;
    const int64_t len = ((n_ctx + (int64_t)d->N + S - 1) / S + 31) / 32 * 32;
    if (len > pl.split_len && (S - 1) * len < n_ctx) pl.split_len = (int)len;
  }
  pl.n_parts = pl.n_ctx_splits + (pl.tree_in_last ? 0 : 1);
  pl.rows = (int64_t)d->B * d->Hq * d->N;
  return pl;
}

// The plan of a call, with the workspace layout shared by both modes: the
// workspace query, the partials and a merge called on its own see the same
// offsets whichever mode ran.  Layout: partial rows [rows][part_stride][D]
// float32, their log2-sum-exps [rows][part_stride], then a 256-byte header
// whose first int32 is the part count the partial kernels used.
va::Plan make_plan(const va_attn_desc* d, int32_t n_ctx, bool sparse) {
  va::Plan pl = plan_cut(d, n_ctx, sparse);
  const int other = plan_cut(d, n_ctx, !sparse).n_parts;
  pl.part_stride = pl.n_parts > other ? pl.n_parts : other;
  const size_t o_bytes = (size_t)pl.rows * pl.part_stride * d->D * sizeof(float);
  pl.off_lse = align_up(o_bytes);
  pl.off_hdr = pl.off_lse + align_up((size_t)pl.rows * pl.part_stride * sizeof(float));
  pl.ws_bytes = pl.off_hdr + 256;
  return pl;
}

float eff_scale(const va_attn_desc* d) { return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->D); }

va_status run_partials(const va_attn_desc* d, const void* q, const void* kc, const void* vc, const void* kd,
                       const void* vd, const int32_t* parent, bool sparse, const int32_t* idx, int32_t K,
                       int64_t idx_stride, void* ws, size_t ws_bytes, hipStream_t stream) {
  va_status st = check_desc(d);
  if (st != VA_OK) return st;
  const int32_t n_ctx = sparse ? K : d->L;
  if (sparse) {
    if (K < 0 || K > d->L) return fail(VA_EINVAL, "K = %d outside [0, L = %d]", K, d->L);
    if (K > 0 && idx == nullptr) return fail(VA_EINVAL, "verify_idx must be non-NULL when K > 0");
    if (K > 0 && idx_stride < K) return fail(VA_EINVAL, "idx_stride (%lld) < K (%d)", (long long)idx_stride, K);
  }
  if (!q || !kd || !vd || !parent) return fail(VA_EINVAL, "q, k_draft, v_draft and parent must be non-NULL");
  if (n_ctx > 0 && (!kc || !vc)) return fail(VA_EINVAL, "k_cache and v_cache must be non-NULL when L > 0");
  if (misaligned(q) || misaligned(kc) || misaligned(vc) || misaligned(kd) || misaligned(vd))
    return fail(VA_EINVAL, "tensor base pointers must be 16-byte aligned");
  const va::Plan pl = make_plan(d, n_ctx, sparse);
  if (ws_bytes < pl.ws_bytes || ws == nullptr)
    return fail(VA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes, ws ? ws_bytes : (size_t)0);
  const int64_t groups = (int64_t)d->B * d->Hkv * pl.row_tiles * pl.n_parts;
  if (groups > 0x7fffffff) return fail(VA_EUNSUPPORTED, "problem too large for one launch");
  const bool gather = sparse && n_ctx > 0;

  va::PartialParams p{};
  p.q = q;
  p.kc = kc;
  p.vc = vc;
  p.kd = kd;
  p.vd = vd;
  p.parent = parent;
  p.idx = gather ? idx : nullptr;
  p.idx_stride = gather ? idx_stride : 0;
  for (int a = 0; a < 3; ++a) {
    p.qs[a] = d->q_stride[a];
    p.kcs[a] = d->kc_stride[a];
    p.vcs[a] = d->vc_stride[a];
    p.kds[a] = d->kd_stride[a];
    p.vds[a] = d->vd_stride[a];
  }
  p.part_o = (float*)ws;
  p.part_lse = (float*)((char*)ws + pl.off_lse);
  p.hdr = (int*)((char*)ws + pl.off_hdr);
  p.B = d->B;
  p.Hq = d->Hq;
  p.Hkv = d->Hkv;
  p.G = d->Hq / d->Hkv;
  p.N = d->N;
  p.L = d->L;
  p.n_ctx = n_ctx;
  p.R = p.G * d->N;
  p.row_tiles = pl.row_tiles;
  p.split_len = pl.split_len;
  p.n_ctx_splits = pl.n_ctx_splits;
  p.n_parts = pl.n_parts;
  p.part_stride = pl.part_stride;
  p.tree_in_last = pl.tree_in_last;
  p.total_groups = (int)groups;
  p.c = eff_scale(d) * 1.4426950408889634f;
  hipError_t e = va::launch_partials(p, d->dtype, d->D, pl.rb, gather, stream);
  if (e != hipSuccess) return fail(VA_EHIP, "partial kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// mode: 0 after dense partials, 1 after sparse ones, -1 unknown (a merge
// called on its own: when the two modes' plans join different part counts,
// the kernel reads the count from the header the partial kernels wrote)
va_status run_merge(const va_attn_desc* d, int32_t n_ctx, void* out, float* lse, const void* ws, size_t ws_bytes,
                    int mode, hipStream_t stream) {
  va_status st = check_desc(d);
  if (st != VA_OK) return st;
  if (n_ctx < 0 || n_ctx > d->L) return fail(VA_EINVAL, "n_ctx = %d outside [0, L]", n_ctx);
  if (!out) return fail(VA_EINVAL, "out must be non-NULL");
  if (misaligned(out)) return fail(VA_EINVAL, "out must be 16-byte aligned");
  const va::Plan pl = make_plan(d, n_ctx, mode == 1);
  if (ws_bytes < pl.ws_bytes || ws == nullptr)
    return fail(VA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes, ws ? ws_bytes : (size_t)0);
  va::MergeParams m{};
  m.part_o = (const float*)ws;
  m.part_lse = (const float*)((const char*)ws + pl.off_lse);
  m.out = out;
  m.lse = lse;
  for (int a = 0; a < 3; ++a) m.os[a] = d->o_stride[a];
  m.rows = pl.rows;
  m.Hq = d->Hq;
  m.N = d->N;
  if (mode >= 0)
    m.n_parts = pl.n_parts;
  else
    m.n_parts = plan_cut(d, n_ctx, true).n_parts == pl.n_parts ? pl.n_parts : 0;
  m.part_stride = pl.part_stride;
  m.hdr = (const int*)((const char*)ws + pl.off_hdr);
  hipError_t e = va::launch_merge(m, d->dtype, d->D, stream);
  if (e != hipSuccess) return fail(VA_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// Fixed device scratch of verify_attn_dense_noalloc: the split partials
// (normalised partial rows and their log2-sum-exps) of one call.  Each GPU
// the library runs on holds its own copy until the process ends; its device
// address is looked up once per device (the name itself is a host-side
// stand-in and is never passed to a kernel or a copy).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev (looked up on the first call on
// that device, with dev current); nullptr and a message on failure.
void* scratch_on(int dev, va_status* st) {
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(VA_EUNSUPPORTED, "device %d beyond the %d devices the fixed scratch serves", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || ptr == nullptr) {
      *st = fail(VA_EHIP, "looking up the fixed scratch on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

va_status verify_attn_dense_noalloc(const va_attn_desc* desc, const void* q, const void* k_cache,
                                    const void* v_cache, const void* k_draft, const void* v_draft,
                                    const int32_t* parent, void* out, float* lse, void* stream) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (!out) return fail(VA_EINVAL, "out must be non-NULL");
  if (misaligned(out)) return fail(VA_EINVAL, "out must be 16-byte aligned");
  const size_t need = make_plan(desc, desc->L, false).ws_bytes;
  if (need > kScratchBytes)
    return fail(VA_EWORKSPACE, "this shape needs %zu bytes of partials, beyond the fixed scratch of %zu bytes "
                "(use verify_attn_dense with a caller workspace)", need, kScratchBytes);
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VA_EHIP, "device of the stream: %s", hipGetErrorString(e));
  void* ws = scratch_on(dev, &st);
  if (ws == nullptr) return st;
  st = run_partials(desc, q, k_cache, v_cache, k_draft, v_draft, parent, false, nullptr, desc->L, 0, ws,
                    kScratchBytes, (hipStream_t)stream);
  if (st != VA_OK) return st;
  return run_merge(desc, desc->L, out, lse, ws, kScratchBytes, 0, (hipStream_t)stream);
}

size_t va_noalloc_scratch_bytes(void) { return kScratchBytes; }

va_status va_attn_workspace_size(const va_attn_desc* desc, int32_t n_ctx, size_t* bytes) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (bytes == nullptr) return fail(VA_EINVAL, "bytes is NULL");
  if (n_ctx < 0 || n_ctx > desc->L) return fail(VA_EINVAL, "n_ctx = %d outside [0, L]", n_ctx);
  *bytes = make_plan(desc, n_ctx, false).ws_bytes;   // the same layout for either mode
  return ok();
}

va_status verify_attn_partials(const va_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                               const void* k_draft, const void* v_draft, const int32_t* parent,
                               const int32_t* verify_idx, int32_t K, int64_t idx_stride, void* ws,
                               size_t ws_bytes, void* stream) {
  return run_partials(desc, q, k_cache, v_cache, k_draft, v_draft, parent, verify_idx != nullptr, verify_idx, K,
                      idx_stride, ws, ws_bytes, (hipStream_t)stream);
}

va_status verify_attn_merge(const va_attn_desc* desc, int32_t n_ctx, void* out, float* lse, const void* ws,
                            size_t ws_bytes, void* stream) {
  return run_merge(desc, n_ctx, out, lse, ws, ws_bytes, -1, (hipStream_t)stream);
}

va_status verify_attn_dense(const va_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                            const void* k_draft, const void* v_draft, const int32_t* parent, void* out,
                            float* lse, void* ws, size_t ws_bytes, void* stream) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (!out) return fail(VA_EINVAL, "out must be non-NULL");
  if (misaligned(out)) return fail(VA_EINVAL, "out must be 16-byte aligned");
  st = run_partials(desc, q, k_cache, v_cache, k_draft, v_draft, parent, false, nullptr, desc->L, 0, ws, ws_bytes,
                    (hipStream_t)stream);
  if (st != VA_OK) return st;
  return run_merge(desc, desc->L, out, lse, ws, ws_bytes, 0, (hipStream_t)stream);
}

va_status verify_attn_sparse(const va_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                             const void* k_draft, const void* v_draft, const int32_t* parent,
                             const int32_t* verify_idx, int32_t K, int64_t idx_stride, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (!out) return fail(VA_EINVAL, "out must be non-NULL");
  if (misaligned(out)) return fail(VA_EINVAL, "out must be 16-byte aligned");
  st = run_partials(desc, q, k_cache, v_cache, k_draft, v_draft, parent, true, verify_idx, K, idx_stride, ws,
                    ws_bytes, (hipStream_t)stream);
  if (st != VA_OK) return st;
  return run_merge(desc, K, out, lse, ws, ws_bytes, 1, (hipStream_t)stream);
}

va_status va_select_workspace_size(int32_t B, int32_t L, size_t* bytes) {
  if (bytes == nullptr) return fail(VA_EINVAL, "bytes is NULL");
  if (B < 0 || L < 0) return fail(VA_EINVAL, "B and L must be >= 0");
  *bytes = va::select_ws_bytes(B, L);
  return ok();
}

va_status select_verify_set(const float* draft_score, const float* target_score, int32_t B, int32_t L, int64_t ld,
                            int32_t sink, int32_t window, int32_t top_m, int32_t budget, int32_t* verify_idx,
                            void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || L < 0) return fail(VA_EINVAL, "B and L must be >= 0");
  if (sink < 0 || window < 0 || top_m < 0 || budget < 0)
    return fail(VA_EINVAL, "sink, window, top_m and budget must be >= 0");
  if (ld < L) return fail(VA_EINVAL, "ld (%lld) < L (%d)", (long long)ld, L);
  const int64_t k_out = budget < L ? budget : L;
  if (B == 0 || k_out == 0) return ok();
  const int64_t sink_n = sink < L ? sink : L;
  const int64_t win_lo = L - (int64_t)(window < L ? window : L);
  const int64_t protected_n = (win_lo > sink_n ? sink_n + (L - win_lo) : L);
  if (budget < L && budget < protected_n)
    return fail(VA_EINVAL, "budget (%d) smaller than sink + window (%lld)", budget, (long long)protected_n);
  if (!verify_idx) return fail(VA_EINVAL, "verify_idx must be non-NULL");
  if (budget < L && L > va::kSelectMaxL)
    return fail(VA_EUNSUPPORTED, "L = %d exceeds the selector limit of %d tokens", L, va::kSelectMaxL);
  if (budget < L && (!draft_score || !target_score))
    return fail(VA_EINVAL, "draft_score and target_score must be non-NULL");
  const size_t need = budget < L ? va::select_ws_bytes(B, L) : 0;
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(VA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : (size_t)0);
  hipError_t e = va::launch_select(draft_score, target_score, B, L, ld, sink, window, top_m, budget, verify_idx, ws,
                                   (hipStream_t)stream);
  if (e != hipSuccess) return fail(VA_EHIP, "select kernel launch: %s", hipGetErrorString(e));
  return ok();
}

va_status accept_commit(const va_attn_desc* desc, void* k_cache, void* v_cache, const void* k_draft,
                        const void* v_draft, const int32_t* parent, const int32_t* accepted, const int32_t* cache_len,
                        int32_t* new_len, void* stream) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (!k_cache || !v_cache || !k_draft || !v_draft || !parent || !accepted || !cache_len || !new_len)
    return fail(VA_EINVAL, "every tensor of accept_commit must be non-NULL");
  // Every workgroup of a sequence reads cache_len[b], accepted[b] and its
  // parent row, while one of them writes new_len[b]: an in-place length
  // update would race with the other KV heads' reads.
  {
    const int64_t nb = (int64_t)desc->B * 4;
    if (overlaps(new_len, nb, cache_len, nb) || overlaps(new_len, nb, accepted, nb) ||
        overlaps(new_len, nb, parent, nb * desc->N))
      return fail(VA_EINVAL, "new_len must not overlap cache_len, accepted or parent");
  }
  if (misaligned(k_cache) || misaligned(v_cache) || misaligned(k_draft) || misaligned(v_draft))
    return fail(VA_EINVAL, "tensor base pointers must be 16-byte aligned");
  va::CommitParams p{};
  p.kc = k_cache;
  p.vc = v_cache;
  p.kd = k_draft;
  p.vd = v_draft;
  p.parent = parent;
  p.accepted = accepted;
  p.cache_len = cache_len;
  p.new_len = new_len;
  for (int a = 0; a < 3; ++a) {
    p.kcs[a] = desc->kc_stride[a];
    p.vcs[a] = desc->vc_stride[a];
    p.kds[a] = desc->kd_stride[a];
    p.vds[a] = desc->vd_stride[a];
  }
  p.B = desc->B;
  p.Hkv = desc->Hkv;
  p.N = desc->N;
  p.capacity = desc->L;
  p.es = desc->dtype == VA_BF16 ? 2 : 4;
  p.row_bytes = desc->D * p.es;
  if ((int64_t)p.B * p.Hkv > 0x7fffffff) return fail(VA_EUNSUPPORTED, "problem too large for one launch");
  hipError_t e = va::launch_commit(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VA_EHIP, "commit kernel launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {

struct ScorePlan {
  int split_len, n_splits;
  int64_t ld_s;
  size_t off_m, off_l, ws_bytes;
};

va_status check_score_desc(const va_score_desc* d) {
  if (d == nullptr) return fail(VA_EINVAL, "desc is NULL");
  if (d->B < 1 || d->Hs < 1) return fail(VA_EINVAL, "B and Hs must be >= 1");
  if (d->L < 0) return fail(VA_EINVAL, "L must be >= 0");
  if (d->M < 1 || d->M > 32) return fail(VA_EUNSUPPORTED, "M = %d query rows per head (supported: 1..32)", d->M);
  if (d->D != 64 && d->D != 128) return fail(VA_EUNSUPPORTED, "D = %d (supported: 64, 128)", d->D);
  if (d->dtype != VA_BF16) return fail(VA_EUNSUPPORTED, "importance scores take bf16 queries and keys");
  if (isnan(d->scale) || isinf(d->scale)) return fail(VA_EINVAL, "scale must be finite");
  for (int a = 0; a < 3; ++a)
    if (d->q_stride[a] % 8 != 0 || d->k_stride[a] % 8 != 0)
      return fail(VA_EINVAL, "q / k strides must keep rows 16-byte aligned");
  if (d->k_stride[2] <= 0) return fail(VA_EUNSUPPORTED, "k token stride must be positive");
  if (((int64_t)d->L + 64) * d->k_stride[2] * 2 > ((int64_t)1 << 31))
    return fail(VA_EUNSUPPORTED, "k: the keys of one (sequence, head) exceed the 2 GiB region limit");
  return VA_OK;
}

ScorePlan make_score_plan(const va_score_desc* d) {
  ScorePlan pl{};
  const int64_t pairs = (int64_t)d->B * d->Hs;
#ifndef VA_SCORE_GROUPS
#define VA_SCORE_GROUPS 256
#endif
  int64_t want = (VA_SCORE_GROUPS + pairs - 1) / pairs;
  if (want < 1) want = 1;
  int64_t len = d->L > 0 ? (d->L + want - 1) / want : 32;
  len = (len + 31) / 32 * 32;
  if (len < 512) len = 512;
  pl.split_len = (int)len;
  pl.n_splits = d->L > 0 ? (int)((d->L + len - 1) / len) : 0;
  pl.ld_s = ((int64_t)d->L + 31) / 32 * 32;
  const int64_t rows = (int64_t)d->B * d->Hs * d->M;
  pl.off_m = align_up((size_t)rows * pl.ld_s * sizeof(float));
  pl.off_l = pl.off_m + align_up((size_t)rows * pl.n_splits * sizeof(float));
  pl.ws_bytes = pl.off_l + align_up((size_t)rows * pl.n_splits * sizeof(float));
  return pl;
}

}  // namespace

va_status va_scores_workspace_size(const va_score_desc* desc, size_t* bytes) {
  va_status st = check_score_desc(desc);
  if (st != VA_OK) return st;
  if (bytes == nullptr) return fail(VA_EINVAL, "bytes is NULL");
  *bytes = make_score_plan(desc).ws_bytes;
  return ok();
}

va_status importance_scores(const va_score_desc* desc, const void* q, const void* k, float* score, int64_t ld_score,
                            void* ws, size_t ws_bytes, void* stream) {
  va_status st = check_score_desc(desc);
  if (st != VA_OK) return st;
  if (!q || !score || (desc->L > 0 && !k)) return fail(VA_EINVAL, "q, k and score must be non-NULL");
  if (misaligned(q) || misaligned(k)) return fail(VA_EINVAL, "q and k must be 16-byte aligned");
  if (ld_score < desc->L) return fail(VA_EINVAL, "ld_score (%lld) < L (%d)", (long long)ld_score, desc->L);
  const ScorePlan pl = make_score_plan(desc);
  if (ws == nullptr || ws_bytes < pl.ws_bytes)
    return fail(VA_EWORKSPACE, "workspace of %zu bytes needed, %zu given", pl.ws_bytes, ws ? ws_bytes : (size_t)0);
  if (desc->L == 0) return ok();
  const int64_t groups = (int64_t)desc->B * desc->Hs * pl.n_splits;
  if (groups > 0x7fffffff) return fail(VA_EUNSUPPORTED, "problem too large for one launch");
  va::ScoreParams p{};
  p.q = q;
  p.k = k;
  for (int a = 0; a < 3; ++a) {
    p.qs[a] = desc->q_stride[a];
    p.ks[a] = desc->k_stride[a];
  }
  p.score = score;
  p.ld_out = ld_score;
  p.s = (float*)ws;
  p.stat_m = (float*)((char*)ws + pl.off_m);
  p.stat_l = (float*)((char*)ws + pl.off_l);
  p.ld_s = pl.ld_s;
  p.B = desc->B;
  p.Hs = desc->Hs;
  p.M = desc->M;
  p.L = desc->L;
  p.split_len = pl.split_len;
  p.n_splits = pl.n_splits;
  p.total_groups = (int)groups;
  const float scale = desc->scale > 0.f ? desc->scale : 1.0f / sqrtf((float)desc->D);
  p.c = scale * 1.4426950408889634f;
  hipError_t e = va::launch_scores(p, desc->D, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VA_EHIP, "score kernel launch: %s", hipGetErrorString(e));
  return ok();
}

va_status verify_set_recovery(const float* score, int64_t ld_score, int32_t B, int32_t L, const int32_t* verify_idx,
                              int32_t K, int64_t idx_stride, int32_t rows, int32_t accumulate, float* arr,
                              void* stream) {
  if (B < 0 || L < 0 || K < 0) return fail(VA_EINVAL, "B, L and K must be >= 0");
  if (rows < 1) return fail(VA_EINVAL, "rows must be >= 1");
  if (ld_score < L) return fail(VA_EINVAL, "ld_score (%lld) < L (%d)", (long long)ld_score, L);
  if (K > 0 && idx_stride < K) return fail(VA_EINVAL, "idx_stride (%lld) < K (%d)", (long long)idx_stride, K);
  if (B == 0) return ok();
  if (!arr || (K > 0 && (!score || !verify_idx))) return fail(VA_EINVAL, "score, verify_idx and arr must be non-NULL");
  if (B > 0x7fffffff) return fail(VA_EUNSUPPORTED, "problem too large for one launch");
  hipError_t e = va::launch_recovery(score, ld_score, B, L, verify_idx, K, idx_stride, rows, accumulate != 0, arr,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(VA_EHIP, "recovery kernel launch: %s", hipGetErrorString(e));
  return ok();
}

va_status build_draft_tree(const float* cand_prob, const int32_t* cand_token, int32_t B, int32_t K, int32_t T,
                           int32_t N, int32_t* parent, int32_t* token, float* rho, float* a_hat, void* stream) {
  if (B < 0) return fail(VA_EINVAL, "B must be >= 0");
  if (K < 1 || T < 1 || N < 1) return fail(VA_EINVAL, "K, T and N must be >= 1");
  if (N > va::kTreeMaxN) return fail(VA_EUNSUPPORTED, "N = %d exceeds %d nodes", N, va::kTreeMaxN);
  if (T > 0xFFFF || (int64_t)K * T > va::kTreeMaxKT)
    return fail(VA_EUNSUPPORTED, "K x T = %lld candidates exceed %d", (long long)K * T, va::kTreeMaxKT);
  // prefixes available: T + T^2 + ... + T^K (saturating)
  int64_t prefixes = 0, level = 1;
  for (int d = 1; d <= K && prefixes < N; ++d) {
    level = level * T > (int64_t)1 << 40 ? (int64_t)1 << 40 : level * T;
    prefixes += level;
  }
  if (prefixes < N) return fail(VA_EINVAL, "only %lld prefixes for N = %d nodes", (long long)prefixes, N);
  if (B == 0) return ok();
  if (!cand_prob || !cand_token || !parent || !token || !rho || !a_hat)
    return fail(VA_EINVAL, "every tensor of build_draft_tree must be non-NULL");
  va::TreeParams p{cand_prob, cand_token, parent, token, rho, a_hat, B, K, T, N};
  hipError_t e = va::launch_tree(p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(VA_EHIP, "tree kernel launch: %s", hipGetErrorString(e));
  return ok();
}

va_status va_verify_time_model(const va_attn_desc* desc, int32_t n_ctx, const va_time_consts* k, int32_t N,
                               double* seconds) {
  va_status st = check_desc(desc);
  if (st != VA_OK) return st;
  if (!seconds || !k) return fail(VA_EINVAL, "consts and seconds must be non-NULL");
  if (n_ctx < 0 || N < 1 || N > 256) return fail(VA_EINVAL, "0 <= n_ctx and 1 <= N <= 256 required");
  if (!(k->bandwidth > 0.0) || !(k->compute_shared > 0.0) || !(k->compute_tiles > 0.0) || !(k->overhead >= 0.0))
    return fail(VA_EINVAL, "bandwidth and compute rates must be > 0, overhead >= 0");
  va_attn_desc d = *desc;
  d.N = N;
  const va::Plan pl = make_plan(&d, n_ctx, false);   // a dense call's plan
  const double e = desc->dtype == VA_BF16 ? 2.0 : 4.0;
  const double B = desc->B, Hq = desc->Hq, Hkv = desc->Hkv, D = desc->D, L = n_ctx;
  const double rows = pl.rb == va::kRowsKernel ? 256.0 : 32.0 * pl.rb;
  const double kv = 2.0 * B * Hkv * L * D * e;
  const double f_pad = 4.0 * B * Hkv * pl.row_tiles * rows * L * D;
  const double w = 2.0 * B * Hq * N * pl.n_parts * (D + 1) * 4.0;
  const double comp = pl.rb == va::kRowsKernel ? k->compute_shared : k->compute_tiles;
  // grid rounds of one context workgroup per CU of the plan's 256-CU target
  const double groups = (double)desc->B * desc->Hkv * pl.row_tiles * pl.n_ctx_splits;
  const double q = groups > 0 ? ceil(groups / VA_TARGET_GROUPS) * VA_TARGET_GROUPS / groups : 1.0;
  const double tb = kv / k->bandwidth, tf = q * f_pad / comp;
  *seconds = (tb > tf ? tb : tf) + w / k->bandwidth + k->overhead;
  return ok();
}

va_status va_choose_tree_size(const float* a_hat_cum, const double* t_verify, int32_t n_max, double t_draft,
                              double l_ar, int32_t* n_best) {
  if (!a_hat_cum || !t_verify || !n_best) return fail(VA_EINVAL, "a_hat_cum, t_verify and n_best must be non-NULL");
  if (n_max < 1) return fail(VA_EINVAL, "n_max must be >= 1");
  if (!(t_draft >= 0.0) || !(l_ar > 0.0)) return fail(VA_EINVAL, "t_draft >= 0 and l_ar > 0 required");
  auto speedup = [&](int n) { return (double)a_hat_cum[n - 1] * l_ar / (t_draft + t_verify[n - 1]); };
  int n = 1;
  while (n < n_max && speedup(n + 1) > speedup(n)) ++n;
  *n_best = n;
  return ok();
}

const char* va_status_str(va_status s) {
  switch (s) {
    case VA_OK: return "ok";
    case VA_EINVAL: return "invalid argument";
    case VA_EUNSUPPORTED: return "unsupported shape or type";
    case VA_EWORKSPACE: return "workspace missing or too small";
    case VA_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* va_last_error(void) { return g_msg; }

int32_t va_version(void) { return 100; }

}  // extern "C"
