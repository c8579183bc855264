/*
 * verify_attn.h -- speculative-verification attention for AMD MI355X (gfx950).
 *
 * C ABI of libverify_attn.so.  Plain pointers and sizes only.
 *
 * What is computed
 * ----------------
 * A target model verifies N draft tokens in one forward pass.  The drafts
 * form a prefix tree given as a parent array (BASTION, "Drafting a
 * Diffusione a Blocchi Basato su Albero": marginal candidates combined into
 * a prefix tree; a chain is the special case of a single draft block, as in
 * the Dustin summary, "Workflow di Verifica").  For every sequence b, query
 * head h (reading KV head h / (Hq / Hkv)) and draft node i, the output row is
 *
 *     out[b,h,i,:] = sum_j softmax(s)_j * value_j,    s_j = scale * <q[b,h,i,:], key_j>
 *     lse[b,h,i]   = ln sum_j exp(s_j)
 *
 * over the key set  C_b  U  anc(i), where
 *   - C_b is the context part: every cached token [0, L) (dense), or the
 *     verify set I_verify = {verify_idx[b, 0..K)} read in place from the
 *     full cache (sparse; Dustin, "Workflow di Verifica" steps 3-4 and
 *     "Significato e Limitazioni": the cache is indexed, not evicted);
 *   - anc(i) is node i and its ancestors among the draft tokens: the tree
 *     mask of the speculative part (LongSpec, "Tree Attention Ibrida").
 * The context part has no mask.  The library computes it as split partial
 * results plus one tree-masked partial and joins them with a log-sum-exp
 * merge, which is exact (LongSpec, "Tree Attention Ibrida", aggregation).
 *
 * select_verify_set builds I_verify per sequence (Dustin, "Aggregazione
 * Ibrida dell'Attenzione"): the attention-sink prefix [0, sink) and the local
 * window [L - window, L) are kept; the remaining budget is filled first by
 * the top min(top_m, remaining) tokens by draft-lookahead score, then by the
 * best remaining tokens by target-historical score.  Ties go to the lower
 * token index; NaN ranks below -inf; -0 equals +0.  Output is ascending.
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees or keeps a pointer past the call.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *   default stream); no call synchronises.  Buffers must stay alive until the
 *   stream has finished the work.
 * - Argument errors are detected on the host before anything is enqueued and
 *   reported as VA_EINVAL / VA_EUNSUPPORTED / VA_EWORKSPACE; nothing runs.
 *   VA_EHIP reports a failed kernel launch; kernels of that call that were
 *   already enqueued may have run.  va_last_error() gives a message for the
 *   last failing call on the calling thread.
 * - Device-side preconditions (parent, verify_idx contents) are not checked
 *   synchronously.  Violations stay memory-safe: a parent outside [-1, i) is
 *   treated as -1; an index outside [0, L) reads no memory outside the cache
 *   (it is skipped, or read as a zero key and value row); the result is then
 *   unspecified (but finite).
 * - Workspace contents need no initialisation and are not preserved.
 *   Concurrent calls must use distinct workspaces.
 * - Calls keep no global mutable state and are thread-safe.
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum va_status {
  VA_OK = 0,
  VA_EINVAL = 1,        /* malformed argument (null pointer, bad size, bad stride) */
  VA_EUNSUPPORTED = 2,  /* well-formed but outside what the kernels implement     */
  VA_EWORKSPACE = 3,    /* workspace missing or smaller than required             */
  VA_EHIP = 4           /* a HIP launch failed                                     */
} va_status;

typedef enum va_dtype {
  VA_FP32 = 0,          /* float32 inputs and output, float32 arithmetic           */
  VA_BF16 = 1           /* bfloat16 inputs and output, float32 accumulation        */
} va_dtype;

/* Shape and layout of one verification problem (one target-model layer).
 *
 *   q        [B, Hq,  N, D]   queries of the draft nodes (after RoPE)
 *   k_cache  [B, Hkv, L, D]   committed context keys     (v_cache alike)
 *   k_draft  [B, Hkv, N, D]   draft-node keys            (v_draft alike)
 *   out      [B, Hq,  N, D]
 *
 * Each tensor is addressed with element strides over its three outer axes
 * (batch, head, row); the innermost (D) stride is 1.  Token-major caches
 * ([B, L, Hkv, D]) are expressed through the strides.  Base pointers and all
 * strides must keep every row 16-byte aligned.  The key (token / node)
 * strides of the four K/V tensors must be positive, and the keys of one
 * (sequence, kv head) plus 64 must span under 2 GiB: (L + 64) x key stride
 * bytes for the cache, (N + 64) x key stride bytes for the draft tensors
 * (else VA_EUNSUPPORTED); the kernels address them with 32-bit offsets. */
typedef struct va_attn_desc {
  int32_t B;            /* sequences, >= 1                                     */
  int32_t Hq;           /* query heads, >= 1, multiple of Hkv                  */
  int32_t Hkv;          /* key/value heads, >= 1                               */
  int32_t D;            /* head dimension: 64 or 128                           */
  int32_t L;            /* committed context length, >= 0 (0: tree part only)  */
  int32_t N;            /* draft nodes per sequence, 1..256                    */
  int32_t dtype;        /* va_dtype of q, caches, drafts and out               */
  float scale;          /* softmax scale; <= 0 selects 1/sqrt(D)               */
  int64_t q_stride[3];  /* q over (b, query head, node)                        */
  int64_t kc_stride[3]; /* k_cache over (b, kv head, token)                    */
  int64_t vc_stride[3]; /* v_cache over (b, kv head, token)                    */
  int64_t kd_stride[3]; /* k_draft over (b, kv head, node)                     */
  int64_t vd_stride[3]; /* v_draft over (b, kv head, node)                     */
  int64_t o_stride[3];  /* out over (b, query head, node)                      */
} va_attn_desc;

/* Workspace bytes needed by verify_attn_dense (n_ctx = L) or
 * verify_attn_sparse (n_ctx = K).  *bytes is set on VA_OK.  A dense and a
 * sparse call of one shape and n_ctx may cut the work differently (bf16
 * with 33..64 query rows per KV head: one 64-row tile per KV head in a
 * dense call, two 32-row tiles in a sparse one; the tree walked by the last
 * context split in a dense call that fills the chip, in its own workgroups
 * in a sparse one); the workspace holds room for either cut, so the size
 * does not depend on the mode. */
va_status va_attn_workspace_size(const va_attn_desc* desc, int32_t n_ctx, size_t* bytes);

/* Dense verification: context part over every cached token [0, L).
 *   parent  [B, N] int32, contiguous; parent[b,i] in [-1, i) (-1: the node
 *           follows the last committed token, which is part of the context)
 *   out     [B, Hq, N, D] in desc->dtype (strides desc->o_stride)
 *   lse     [B, Hq, N] float32 contiguous, natural log; may be NULL
 *   ws      device workspace of at least va_attn_workspace_size(desc, L) bytes */
va_status verify_attn_dense(const va_attn_desc* desc,
                            const void* q, const void* k_cache, const void* v_cache,
                            const void* k_draft, const void* v_draft,
                            const int32_t* parent,
                            void* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream);

/* verify_attn_dense without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a fixed
 * device array of va_noalloc_scratch_bytes() (64 MiB) that the library
 * holds on each GPU it runs on until the process ends; the call allocates
 * nothing.  Shapes whose partials need more than that return VA_EWORKSPACE
 * (use verify_attn_dense).  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (several streams, or threads)
 * race and must be serialised by the caller.  The device is the stream's
 * (the current device for a NULL stream).  Other arguments as for
 * verify_attn_dense; results are bitwise those of verify_attn_dense. */
va_status verify_attn_dense_noalloc(const va_attn_desc* desc,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    const void* k_draft, const void* v_draft,
                                    const int32_t* parent,
                                    void* out, float* lse, void* stream);

/* Size in bytes of the fixed scratch of verify_attn_dense_noalloc. */
size_t va_noalloc_scratch_bytes(void);

/* Sparse verification: context part over the verify set only.
 *   verify_idx  [B, K] int32, row stride idx_stride (>= K); each row holds K
 *               distinct token positions in [0, L) (any order; ascending is
 *               fastest).  0 <= K <= L.
 * Other arguments as for verify_attn_dense; ws needs
 * va_attn_workspace_size(desc, K) bytes. */
va_status verify_attn_sparse(const va_attn_desc* desc,
                             const void* q, const void* k_cache, const void* v_cache,
                             const void* k_draft, const void* v_draft,
                             const int32_t* parent,
                             const int32_t* verify_idx, int32_t K, int64_t idx_stride,
                             void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* The two stages that verify_attn_dense / verify_attn_sparse enqueue, for
 * callers that time or schedule them separately.  verify_attn_partials
 * writes the split context partials and the tree partial into ws (the
 * last context split walks the tree after its context keys, and no
 * separate tree partial is written, in the shared-tile kernel whenever the
 * context has splits, and in a dense call whose context workgroups number
 * at least 256)
 * (verify_idx == NULL: dense over [0, L) and K is ignored; otherwise sparse
 * over the K indices); verify_attn_merge joins them into out / lse.  The
 * merge must be given the same desc and ws and n_ctx = L (dense) or K
 * (sparse), and must run after the partials on the stream: where the dense
 * and sparse cuts of the shape join different part counts, it reads the
 * count the partials wrote into ws. */
va_status verify_attn_partials(const va_attn_desc* desc,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* k_draft, const void* v_draft,
                               const int32_t* parent,
                               const int32_t* verify_idx, int32_t K, int64_t idx_stride,
                               void* ws, size_t ws_bytes, void* stream);
va_status verify_attn_merge(const va_attn_desc* desc, int32_t n_ctx,
                            void* out, float* lse,
                            const void* ws, size_t ws_bytes, void* stream);

/* Best-first draft tree (BASTION, "Drafting a Diffusione a Blocchi Basato su
 * Albero" and "Surrogato di Accettazione ed Espansione Best-First").  A block
 * drafter proposes, for each of K positions, T candidate tokens with their
 * marginal probabilities.  A node at depth d picks one candidate at each of
 * the first d positions; its path score is rho = q_0 * ... * q_{d-1}
 * (float32, in that order).  The tree is grown by adding, N times, the valid
 * node of highest rho (the root's best candidate first; adding a node makes
 * its best child and its next sibling valid); ties go to the node whose
 * parent entered first, then to the better-ranked candidate.  Candidates of
 * a position are ranked by probability, ties to the lower candidate index;
 * NaN or negative probabilities count as 0.
 *   cand_prob   [B, K, T] float32 device, contiguous
 *   cand_token  [B, K, T] int32 device, contiguous (token ids, copied out)
 *   parent      [B, N] int32 device, written: node index (< own index) or -1
 *   token       [B, N] int32 device, written: the node's token
 *   rho         [B, N] float32 device, written: non-increasing per sequence
 *   a_hat       [B] float32 device, written: sum of rho in node order (the
 *               surrogate of the expected accepted length)
 * 1 <= N <= 256, K x T <= 4096, and T + T^2 + ... + T^K >= N (else
 * VA_EINVAL / VA_EUNSUPPORTED).  The parent array feeds verify_attn_*. */
va_status build_draft_tree(const float* cand_prob, const int32_t* cand_token, int32_t B,
                           int32_t K, int32_t T, int32_t N, int32_t* parent, int32_t* token,
                           float* rho, float* a_hat, void* stream);

/* Tree-budget controller (BASTION, "Controllore Online del Budget
 * Consapevole dell'Hardware"): a roofline estimate of the verification
 * latency and the rule that sizes the draft tree.  Host functions; no GPU
 * work.
 *
 * va_verify_time_model: T_verify(N) in seconds for desc's shape with N draft
 * nodes over n_ctx context keys, following the plan this library runs (the
 * pages fit the model's constants to measured run times; its structure
 * here is the kernels', those of a dense call): with R = (Hq / Hkv) N query
 * rows per KV head cut into row tiles of `rows` rows (256 in the shared-tile
 * kernel: bf16 with R > 64; else 64 when R > 32, else 32) and the context
 * cut into the call's splits (parts = splits + 1 for the tree, or splits when the
 * last split walks the tree: in the shared-tile kernel, or when the
 * context workgroups number at least 256),
 *     T = max(KV / bandwidth, Q F_pad / compute_k) + W / bandwidth + overhead
 * KV = 2 B Hkv n_ctx D e, F_pad = 4 B Hkv tiles rows n_ctx D (padded rows
 * included), compute_k = compute_shared or compute_tiles by kernel,
 * Q = ceil(Wg / 256) 256 / Wg for the Wg = B Hkv tiles splits context
 * workgroups (grid rounds on 256 CUs, one workgroup each), W = 2 B Hq N
 * parts (D + 1) 4 (partial rows written and merged), e = element bytes.
 * The constants are effective ones calibrated from measured runs (they
 * absorb fixed per-call costs); desc->N is ignored. */
typedef struct {
  double bandwidth;       /* bytes / s                                          */
  double compute_shared;  /* flop / s of the shared-tile kernel (padded rows)   */
  double compute_tiles;   /* flop / s of the per-wavefront kernel (padded rows) */
  double overhead;        /* seconds per call                                   */
} va_time_consts;
va_status va_verify_time_model(const va_attn_desc* desc, int32_t n_ctx, const va_time_consts* consts,
                               int32_t N, double* seconds);

/* va_choose_tree_size: the tree stops growing when the estimated speedup
 * S(n) = a_hat_cum[n-1] * l_ar / (t_draft + t_verify[n-1]) stops increasing:
 * *n_best = the first n with S(n+1) <= S(n), or n_max.  a_hat_cum[n-1] is the
 * surrogate of the best-first tree of n nodes (prefix sums of
 * build_draft_tree's rho), t_verify[n-1] the (estimated) verification time
 * of n nodes, t_draft the drafter's time, l_ar one autoregressive step's
 * time (seconds).  Host pointers. */
va_status va_choose_tree_size(const float* a_hat_cum, const double* t_verify, int32_t n_max,
                              double t_draft, double l_ar, int32_t* n_best);

/* Importance scores for the selector (Dustin, "Metodologia" sections 1-2:
 * attention scores of a few scoring heads -- the draft's lookahead rows or
 * the target's previous rows -- aggregated into one global importance map):
 *
 *     score[b, j] = sum_{h < Hs} sum_{i < M} softmax_j(scale * <q[b,h,i], k[b,h,j]>)
 *
 * with the softmax over the L context tokens (the pages leave the
 * aggregation open; the plain reading is this sum of probabilities).  The
 * result is what select_verify_set takes as draft_score or target_score. */
typedef struct {
  int32_t B;            /* sequences                                          */
  int32_t Hs;           /* scoring heads                                      */
  int32_t M;            /* query rows per scoring head, 1..32                 */
  int32_t D;            /* head dimension, 64 or 128                          */
  int32_t L;            /* context tokens, >= 0                               */
  int32_t dtype;        /* VA_BF16 only                                       */
  float scale;          /* softmax scale; <= 0 selects 1/sqrt(D)              */
  int64_t q_stride[3];  /* q [B, Hs, M, D] over (b, head, row), unit D stride */
  int64_t k_stride[3];  /* k [B, Hs, L, D] over (b, head, token); token stride
                           > 0, (L + 64) x token stride x 2 bytes <= 2 GiB    */
} va_score_desc;

/* Workspace bytes importance_scores needs for this desc (about
 * 4 x B x Hs x M x L bytes: the scaled scores between its two kernels). */
va_status va_scores_workspace_size(const va_score_desc* desc, size_t* bytes);

/* score [B, L] float32 device, row stride ld_score (>= L), written.  q and
 * k device pointers, 16-byte aligned; ws device workspace of
 * va_scores_workspace_size bytes.  Two kernels on `stream`. */
va_status importance_scores(const va_score_desc* desc, const void* q, const void* k,
                            float* score, int64_t ld_score,
                            void* ws, size_t ws_bytes, void* stream);

/* Attention Recovery Rate of a verify set (Dustin, "Metodologia" section 2
 * names it as the objective of the offline choice of scoring heads and of
 * m; the pages give no formula).  Reading: the share of the full context
 * attention mass of the verification rows that the set keeps,
 *     arr[b] = (1 / rows) sum_{k < K} score[b, verify_idx[b, k]]
 * where score is importance_scores' map over ALL `rows` query rows of the
 * verification (every query head's draft rows, each against its KV head),
 * so arr = 1 for the whole cache.  That map may come in pieces (one
 * importance_scores call takes up to 32 rows of one KV head): with
 * accumulate != 0 the piece's share is added to arr instead of written.
 *   score       [B, L] float32 device, row stride ld_score (>= L)
 *   verify_idx  [B, K] int32 device, row stride idx_stride (>= K), distinct
 *               indices (duplicates count twice; indices outside [0, L) add 0)
 *   arr         [B] float32 device, written
 * One kernel on `stream`; the sum order is fixed (bitwise reproducible). */
va_status verify_set_recovery(const float* score, int64_t ld_score, int32_t B, int32_t L,
                              const int32_t* verify_idx, int32_t K, int64_t idx_stride,
                              int32_t rows, int32_t accumulate, float* arr, void* stream);

/* Accept and commit (Dustin, "Workflow di Verifica" step 5: accepted draft
 * tokens are appended to the cache, rejected ones dropped).  The accepted
 * tokens of sequence b are the root-to-node path of the draft tree that ends
 * at node accepted[b]; their K/V rows (every KV head) are copied, root
 * first, from k_draft / v_draft to positions cache_len[b], cache_len[b] + 1,
 * ... of k_cache / v_cache, and new_len[b] = cache_len[b] + path length.
 *   desc        as for verify_attn_dense, with desc->L = the cache capacity
 *               (token rows allocated per (sequence, kv head)); q / out
 *               fields are not used
 *   k_cache, v_cache  [B, Hkv, capacity, D], written in place
 *   parent      [B, N] as for verify_attn_dense
 *   accepted    [B] int32 device: deepest accepted node in [0, N), or -1 for
 *               none (values outside [-1, N) act as -1)
 *   cache_len   [B] int32 device: valid tokens per sequence before the call
 *   new_len     [B] int32 device, written; it must not overlap cache_len,
 *               accepted or parent (VA_EINVAL): every KV head's workgroup
 *               reads those while one of them writes new_len, so an
 *               in-place length update would race.  Update the lengths by
 *               copying new_len into cache_len after the call.
 * Rows that would land at or past the capacity are not written (new_len
 * still counts them).  Device pointers, asynchronous on `stream`; no
 * workspace.  Malformed parents end a path as in the tree mask. */
va_status accept_commit(const va_attn_desc* desc, void* k_cache, void* v_cache,
                        const void* k_draft, const void* v_draft, const int32_t* parent,
                        const int32_t* accepted, const int32_t* cache_len, int32_t* new_len,
                        void* stream);

/* Workspace bytes needed by select_verify_set for B rows of L scores when
 * it selects (budget < L): per row, about 6 bytes per token for the
 * candidate lists its first kernel writes and its second reads.  Calls that
 * overlap in time must not share a workspace. */
va_status va_select_workspace_size(int32_t B, int32_t L, size_t* bytes);

/* Verify-set selection.
 *   draft_score, target_score  [B, L] float32, row stride ld (>= L)
 *   sink, window, top_m >= 0; budget >= min(L, |[0,sink) U [L-window,L)|)
 *   verify_idx  [B, min(budget, L)] int32, contiguous; ascending, distinct
 *   ws          device workspace of va_select_workspace_size(B, L) bytes
 *               (unused, and may be NULL, when budget >= L)
 * budget >= L returns every index 0..L-1.  With budget < L, rows longer
 * than 786432 tokens (24 x 32768) return VA_EUNSUPPORTED: a row whose
 * sample misses is resolved by one workgroup that re-reads the row on
 * every radix pass, and the limit bounds that time.
 * Two kernels run on `stream`: a filter over 4096-token workgroups that
 * lists, per row, every token either tier could take (key bounds from a
 * row-wide sample), then one workgroup per row that finds both thresholds
 * exactly among the listed tokens (or over the whole row when the list
 * cannot hold them) and writes the verify set.  Neither waits on another
 * workgroup. */
va_status select_verify_set(const float* draft_score, const float* target_score,
                            int32_t B, int32_t L, int64_t ld,
                            int32_t sink, int32_t window, int32_t top_m, int32_t budget,
                            int32_t* verify_idx,
                            void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* va_status_str(va_status status);

/* Message describing the last failing call on this thread ("" if none). */
const char* va_last_error(void);

/* Library version, as MAJOR * 10000 + MINOR * 100 + PATCH. */
int32_t va_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
