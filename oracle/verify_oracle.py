"""CPU oracle for speculative-verification attention and verify-set selection.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the benchmark's CPU-baseline leg may import this module.  The HIP library
never calls it and shares no code with it.

Everything is plain numpy in float64, written for a reader to check against
the pages by eye:

* ``verify_attention`` is the plain definition of what the hybrid tree
  attention computes (LongSpec, "Tree Attention Ibrida"): each draft node
  attends, with no mask, to every context key (the whole cache, or the
  verify subset of Dustin, "Workflow di Verifica" steps 3-4), and, under the
  tree mask, to itself and its ancestors among the draft nodes.  The page
  splits the two parts and re-joins them with a log-sum-exp merge; that merge
  is exact, so its result is the single softmax over the concatenated key set
  that is written out here.  No split, no merge, no blocking.
* ``accept_commit`` is the last step of the verification workflow (Dustin,
  "Workflow di Verifica" step 5): the accepted draft tokens are appended to
  the cache and the rejected ones dropped.  The accepted tokens of a
  sequence are a path of the draft tree from a root to its deepest accepted
  node; their K/V rows are written, root first, at the sequence's current
  cache length.
* ``importance_scores`` produces the per-token scores the selector ranks
  (Dustin, "Metodologia" sections 1-2: attention scores of the target's
  previous passes and of the draft's lookahead, computed on a few selected
  heads only, aggregated into one global importance map).  The pages do not
  spell the aggregation out; the plain reading taken here is the sum, over
  the scoring heads and their query rows, of the attention probabilities
  each row gives to every context token.
* ``best_first_tree`` builds the draft tree the verification takes
  (BASTION, "Drafting a Diffusione a Blocchi Basato su Albero" and
  "Surrogato di Accettazione ed Espansione Best-First"): from per-position
  candidate tokens with their marginal probabilities it adds, N times, the
  valid node (a child of the tree or of the root) with the highest path score
  rho = product of the marginals along the path.
* ``verify_time_model`` and ``choose_tree_size`` follow BASTION's online
  budget controller ("Controllore Online del Budget Consapevole
  dell'Hardware"): a roofline estimate of the verification latency,
  T_verify(N) = max(bytes(N) / bandwidth, flops(N) / compute) + overhead,
  with the three constants calibrated from measured runs, and a stopping
  rule that grows the tree while the estimated speedup
  S(N) = A_hat(N) * L_AR / C(N) still increases.
* ``select_verify_set`` follows the selection rule of Dustin, "Metodologia"
  section 1 (Aggregazione Ibrida dell'Attenzione): protect an attention-sink
  prefix and a local window of recent tokens, then fill the remaining budget
  with the top-m tokens by the draft-lookahead score, then the most relevant
  remaining tokens by the target-historical score.  It is written with a
  stable sort.

Readings where the pages are silent (each listed with its reason in the
design notes of the repository):

* softmax scale 1/sqrt(D); query head h reads KV head h // (Hq // Hkv);
* ``parent[i] == -1`` means node i hangs off the last committed token, which
  is already in the context; ``parent[i] < i`` (topological order);
* the verify set restricts the context part only, the draft part is always
  complete; the budget counts the sink and the window; sink and window are a
  union; the draft tier takes min(m, remaining budget, remaining tokens);
* ties in a score go to the lower token index; NaN ranks below -inf, and
  -0 equals +0; the output index list is ascending;
* ``lse`` is the natural-log log-sum-exp of the scaled scores of a row;
* importance scores: the softmax of a scoring row runs over the context
  tokens [0, L) only, and the map is the plain sum of the probabilities;
* draft tree: position k's candidates are ranked by probability (ties: lower
  candidate index); rho is accumulated in float32, parent first; equal rho
  goes to the node whose parent entered the tree first, then to the better
  ranked candidate; probabilities that are NaN or negative count as 0; the
  expected acceptance surrogate is the float32 sum of rho in node order;
* budget controller: C(N) = T_draft + T_verify(N) (the drafter's cost does
  not depend on the tree shape), L_AR is the latency of one autoregressive
  step, and "starts to decrease" means the tree stops at the first N with
  S(N + 1) <= S(N).

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, textbook special cases, brute force); none is "parity
unpinned".
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# inputs


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 view of an input tensor (bf16 bits or float32)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# tree mask (LongSpec "Tree Attention Ibrida": the speculative part needs the
# tree mask; BASTION "Drafting a Diffusione a Blocchi Basato su Albero": the
# candidates form a prefix tree)


def ancestor_mask(parent: Sequence[int]) -> np.ndarray:
    """anc[i, j] is True when draft node j is node i or one of its ancestors.

    Built by walking each node's parent chain up to the virtual root (-1).
    """
    parent = [int(p) for p in parent]
    n = len(parent)
    anc = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if not -1 <= parent[i] < i:
            raise ValueError(f"parent[{i}] = {parent[i]} breaks -1 <= parent[i] < i")
        j = i
        while j != -1:
            anc[i, j] = True
            j = parent[j]
    return anc


# ---------------------------------------------------------------------------
# attention


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     mask: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of rows q[R, D] over keys k[C, D] / values v[C, D].

    mask[R, C] marks the keys each row may see.  One softmax per row over all
    its visible keys, max-subtracted.  Returns (out[R, D], lse[R]) with
    lse = ln(sum_j exp(s_j)) over the visible keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    if not mask.any(axis=1).all():
        raise ValueError("a row sees no key")
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def default_scale(D: int) -> float:
    return 1.0 / np.sqrt(D)


def verify_attention(q, k_cache, v_cache, k_draft, v_draft, parent,
                     scale: Optional[float] = None,
                     ctx_index: Optional[np.ndarray] = None,
                     heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Verification attention of N draft nodes against the target KV cache.

    Shapes: q [B, Hq, N, D]; k_cache, v_cache [B, Hkv, L, D];
    k_draft, v_draft [B, Hkv, N, D]; parent [B, N] int.  Inputs may be bf16
    bit patterns (uint16) or floats; they are upcast exactly to float64.

    ctx_index [B, K]: when given, sequence b's context part is the key set
    {ctx_index[b, :]} (Dustin's verify set, read from the full cache in place)
    instead of the whole cache [0, L).

    heads: optional (b, h) pairs; then only those are computed and the result
    is (out[len(heads), N, D], lse[len(heads), N]).  Otherwise the result is
    (out[B, Hq, N, D], lse[B, Hq, N]).
    """
    B, Hq, N, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    L = k_cache.shape[2]
    sc = default_scale(D) if scale is None else float(scale)
    pairs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]

    outs = np.empty((len(pairs), N, D), dtype=np.float64)
    lses = np.empty((len(pairs), N), dtype=np.float64)
    anc_cache = {}
    kv_cache = {}
    for n, (b, h) in enumerate(pairs):
        if b not in anc_cache:
            anc_cache[b] = ancestor_mask(parent[b])
        anc = anc_cache[b]
        kv = h // G
        if (b, kv) not in kv_cache:
            kv_cache.clear()
            if ctx_index is None:
                pos = np.arange(L)
            else:
                pos = np.unique(np.asarray(ctx_index[b], dtype=np.int64))
                if pos.size and (pos[0] < 0 or pos[-1] >= L):
                    raise ValueError("ctx_index out of range")
            keys = np.concatenate([as_f64(k_cache[b, kv][pos]), as_f64(k_draft[b, kv])])
            vals = np.concatenate([as_f64(v_cache[b, kv][pos]), as_f64(v_draft[b, kv])])
            kv_cache[(b, kv)] = (pos.size, keys, vals)
        C, keys, vals = kv_cache[(b, kv)]
        mask = np.concatenate([np.ones((N, C), dtype=bool), anc], axis=1)
        o, l = masked_attention(as_f64(q[b, h]), keys, vals, mask, sc)
        outs[n] = o
        lses[n] = l
    if heads is not None:
        return outs, lses
    return outs.reshape(B, Hq, N, D), lses.reshape(B, Hq, N)


# ---------------------------------------------------------------------------
# verify-set selection (Dustin, "Aggregazione Ibrida dell'Attenzione")


def _rank_order(score: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """Candidates sorted best first: higher score first, lower index on ties.

    NaN ranks below every number (also below -inf); -0 and +0 are equal.
    """
    s = np.asarray(score, dtype=np.float64)[cand]
    is_num = ~np.isnan(s)
    val = np.where(is_num, s, 0.0) + 0.0    # + 0.0 turns -0 into +0
    # np.lexsort sorts by the last key first, ascending.
    order = np.lexsort((cand, -val, ~is_num))
    return cand[order]


def protected_set(L: int, sink: int, window: int) -> np.ndarray:
    """Attention-sink prefix [0, sink) united with the local window [L-window, L)."""
    sink_part = np.arange(0, min(max(sink, 0), L))
    win_part = np.arange(max(0, L - max(window, 0)), L)
    return np.union1d(sink_part, win_part).astype(np.int64)


def select_row(draft: np.ndarray, target: np.ndarray, sink: int, window: int,
               top_m: int, budget: int) -> np.ndarray:
    L = draft.shape[0]
    if budget >= L:
        return np.arange(L, dtype=np.int64)
    prot = protected_set(L, sink, window)
    if budget < prot.size:
        raise ValueError("budget smaller than sink + window")
    rest_budget = budget - prot.size
    free = np.setdiff1d(np.arange(L), prot)
    m = min(max(top_m, 0), rest_budget, free.size)
    by_draft = _rank_order(draft, free)[:m]
    remaining = np.setdiff1d(free, by_draft)
    by_target = _rank_order(target, remaining)[:rest_budget - m]
    return np.sort(np.concatenate([prot, by_draft, by_target]))


def select_verify_set(draft_score: np.ndarray, target_score: np.ndarray,
                      sink: int, window: int, top_m: int, budget: int) -> np.ndarray:
    """I_verify per sequence: int64 [B, min(budget, L)], ascending."""
    draft_score = np.asarray(draft_score)
    target_score = np.asarray(target_score)
    rows = [select_row(draft_score[b], target_score[b], sink, window, top_m, budget)
            for b in range(draft_score.shape[0])]
    return np.stack(rows) if rows else np.zeros((0, 0), dtype=np.int64)


# ---------------------------------------------------------------------------
# accept and commit


def accepted_path(parent: Sequence[int], leaf: int) -> list:
    """Draft nodes from the root down to ``leaf`` (empty when leaf == -1).

    The accepted tokens of a speculative step form one root-to-node path of
    the draft tree (a node is only accepted after its parent); the path is
    read off the parent array, root first.
    """
    parent = [int(x) for x in parent]
    if leaf == -1:
        return []
    if not 0 <= leaf < len(parent):
        raise ValueError(f"accepted node {leaf} outside [-1, {len(parent)})")
    path = []
    j = leaf
    while j != -1:
        if not -1 <= parent[j] < j:
            raise ValueError(f"parent[{j}] = {parent[j]} breaks -1 <= parent[i] < i")
        path.append(j)
        j = parent[j]
    return path[::-1]


def accept_commit(k_cache: np.ndarray, v_cache: np.ndarray, k_draft: np.ndarray, v_draft: np.ndarray,
                  parent: np.ndarray, accepted: Sequence[int], cache_len: Sequence[int]):
    """Append each sequence's accepted draft path to its cache (Dustin,
    "Workflow di Verifica" step 5).

    k_cache/v_cache [B, Hkv, capacity, D] hold cache_len[b] valid tokens of
    sequence b; the K/V rows of the accepted path's nodes (all KV heads) go
    to positions cache_len[b], cache_len[b] + 1, ... in root-to-leaf order.
    Rows that would land at or past the capacity are dropped.  Returns new
    copies of the caches and new_len[b] = cache_len[b] + path length.
    Element values are copied bit for bit (any dtype).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    capacity = kc.shape[2]
    new_len = np.array(cache_len, dtype=np.int64).copy()
    for b in range(kc.shape[0]):
        path = accepted_path(parent[b], int(accepted[b]))
        for depth, node in enumerate(path):
            pos = int(cache_len[b]) + depth
            if pos < capacity:
                kc[b, :, pos, :] = k_draft[b, :, node, :]
                vc[b, :, pos, :] = v_draft[b, :, node, :]
        new_len[b] = int(cache_len[b]) + len(path)
    return kc, vc, new_len


# ---------------------------------------------------------------------------
# importance scores


def importance_scores(q: np.ndarray, k: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Global importance map [B, L] from a few scoring heads (Dustin,
    "Metodologia" sections 1-2).

    q [B, Hs, M, D]: the query rows of the scoring heads (draft lookahead
    rows, or the target's previous rows); k [B, Hs, L, D]: the context keys
    each scoring head reads.  score[b, j] = sum over h < Hs and i < M of
    softmax_j(scale * <q[b, h, i], k[b, h, j]>), the softmax taken over the
    L context tokens.
    """
    qf, kf = as_f64(q), as_f64(k)
    B, Hs, M, D = qf.shape
    L = kf.shape[2]
    if scale is None or scale <= 0:
        scale = default_scale(D)
    out = np.zeros((B, L), dtype=np.float64)
    for b in range(B):
        for h in range(Hs):
            s = scale * (qf[b, h] @ kf[b, h].T)              # [M, L]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b] += (p / p.sum(axis=1, keepdims=True)).sum(axis=0)
    return out


def attention_recovery(q: np.ndarray, k_cache: np.ndarray, verify_idx: np.ndarray,
                       scale: Optional[float] = None) -> np.ndarray:
    """Attention Recovery Rate of a verify set per sequence (Dustin,
    "Metodologia" section 2 names it as the objective of the offline choice
    of scoring heads; the pages give no formula).  Plain reading: the share
    of the full attention mass that the verify set keeps, i.e. for sequence
    b the mean over query heads h and draft rows i of

        sum_{j in I_verify[b]} softmax_j(scale * <q[b,h,i], k_cache[b, h // G, j]>)

    with the softmax over the L context keys (the draft keys are never
    dropped, so they are not part of it).  q [B, Hq, N, D], k_cache
    [B, Hkv, L, D], verify_idx [B, K] (a set: duplicates count once).
    Returns float64 [B]; an empty set recovers 0."""
    qf, kf = as_f64(q), as_f64(k_cache)
    B, Hq, N, D = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    out = np.zeros(B, dtype=np.float64)
    for b in range(B):
        sel = np.unique(np.asarray(verify_idx[b], dtype=np.int64))
        total = 0.0
        for h in range(Hq):
            s = sc * (qf[b, h] @ kf[b, h // G].T)            # [N, L]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            total += p[:, sel].sum()
        out[b] = total / (Hq * N)
    return out


# ---------------------------------------------------------------------------
# best-first draft tree


def best_first_tree(cand_prob: np.ndarray, cand_token: np.ndarray, N: int):
    """Best-first prefix tree of N draft nodes for one sequence (BASTION,
    "Surrogato di Accettazione ed Espansione Best-First").

    cand_prob, cand_token [K, T]: the T candidate tokens of each of the K
    block positions and their marginal probabilities q_k.  A node at depth d
    is a choice of one candidate at each of positions 0..d-1; its path score
    is rho = q_0 * ... * q_{d-1} (float32, in that order).  Starting from an
    empty tree whose only valid node is the best candidate of position 0,
    each step adds the valid node of highest rho; adding a node makes valid
    its best child (next position) and its next sibling (same parent, next
    candidate of the same position).  Returns parent [N] (-1: child of the
    committed context), token [N], rho [N] (float32) and the surrogate
    A_hat = sum of rho (float32, node order).
    """
    cand_prob = np.asarray(cand_prob, dtype=np.float32)
    K, T = cand_prob.shape
    prob = np.where(cand_prob > 0, cand_prob, np.float32(0))     # NaN and negatives count as 0
    order = [np.lexsort((np.arange(T), -prob[k].astype(np.float64))) for k in range(K)]
    q = np.stack([prob[k][order[k]] for k in range(K)])          # [K, T], descending per position
    tok = np.stack([np.asarray(cand_token)[k][order[k]] for k in range(K)])
    if sum(T ** d for d in range(1, K + 1)) < N:
        raise ValueError("fewer prefixes than N")
    import heapq
    one = np.float32(1.0)
    # heap entries: (-rho, parent node (-1 first), rank, depth, rho of the parent)
    heap = [(-float(q[0, 0]), -1, 0, 1, one)]
    parent, token, rho = [], [], []
    while len(parent) < N:
        neg, par, rank, depth, rho_par = heapq.heappop(heap)
        node = len(parent)
        r = np.float32(rho_par * q[depth - 1, rank])
        parent.append(par)
        token.append(int(tok[depth - 1, rank]))
        rho.append(r)
        if depth < K:                                    # best child
            c = np.float32(r * q[depth, 0])
            heapq.heappush(heap, (-float(c), node, 0, depth + 1, r))
        if rank + 1 < T:                                 # next sibling
            sib = np.float32(rho_par * q[depth - 1, rank + 1])
            heapq.heappush(heap, (-float(sib), par, rank + 1, depth, rho_par))
    a_hat = np.float32(0)
    for r in rho:
        a_hat = np.float32(a_hat + r)
    return (np.array(parent, dtype=np.int32), np.array(token, dtype=np.int32),
            np.array(rho, dtype=np.float32), a_hat)


# ---------------------------------------------------------------------------
# budget controller (BASTION, "Controllore Online del Budget Consapevole
# dell'Hardware")


def verify_bytes_flops(B: int, Hq: int, Hkv: int, D: int, n_ctx: int, N: int, elem_bytes: int):
    """Bytes one verification must move and flops it must do: the K/V rows
    of the context once, the queries, the draft K/V rows, the output and its
    log-sum-exp; 4 flops per (query row, context key, dimension)."""
    kv = 2 * B * Hkv * n_ctx * D * elem_bytes
    q = B * Hq * N * D * elem_bytes
    draft = 2 * B * Hkv * N * D * elem_bytes
    out = B * Hq * N * D * elem_bytes + B * Hq * N * 4
    return kv + q + draft + out, 4 * B * Hq * N * n_ctx * D


def verify_time_model(B: int, Hq: int, Hkv: int, D: int, n_ctx: int, N: int, elem_bytes: int,
                      bandwidth: float, compute: float, overhead: float) -> float:
    """Roofline estimate of T_verify(N) in seconds with calibrated constants."""
    nbytes, flops = verify_bytes_flops(B, Hq, Hkv, D, n_ctx, N, elem_bytes)
    return max(nbytes / bandwidth, flops / compute) + overhead


def kernel_plan(B: int, Hq: int, Hkv: int, n_ctx: int, N: int, elem_bytes: int, sparse: bool = False):
    """How the verification library cuts one call into work (its documented
    plan, restated here): the G * N query rows of a KV head go in row tiles
    of 256 rows (the shared-tile kernel, bf16 with more than 64 rows), else
    for bf16 one 64-row tile (33 to 64 rows in a dense call) or 32-row tiles,
    else 32 or 64 rows (fp32, 64 when more than 32 rows);
    the context keys go in splits of a multiple of 128 keys (at least 512),
    their count chosen for the soonest end of the context workgroups' rounds
    on a 256-CU device running one workgroup per CU.
    The tree is one more part, except where the last context split walks
    the tree after its context keys: in the shared-tile kernel, and in a
    dense call whose context workgroups number at least 256 (one part when
    there is no context).  Returns (shared_tile_kernel, rows per tile, row
    tiles per KV head, context splits, parts)."""
    R = (Hq // Hkv) * N
    shared = elem_bytes == 2 and R > 64
    if shared:
        rows = 256
    elif elem_bytes == 2:
        rows = 64 if R > 32 and not sparse else 32
    elif R <= 32:
        rows = 32
    else:
        rows = 64
    tiles = -(-R // rows)
    pairs = B * Hkv * tiles
    # context splits: of 1 .. 2 s0 splits (s0 the fewest that make 256
    # workgroups), the count whose rounds of 256 workgroups end first
    # (rounds times keys per split), the fewest on a tie
    s0 = -(-256 // pairs) if pairs < 256 else 1
    splits, best = 0, None
    for s in range(1, 2 * s0 + 1) if n_ctx > 0 else ():
        per = -(-n_ctx // s)                        # ceil(n_ctx / s)
        split = max(512, -(-per // 128) * 128)      # a multiple of 128, >= 512
        cnt = -(-n_ctx // split)
        cost = -(-(pairs * cnt) // 256) * split
        if best is None or cost < best:
            best, splits = cost, cnt
    folded = splits > 0 and (shared or (not sparse and pairs * splits >= 256))
    return shared, rows, tiles, splits, splits if folded else splits + 1


def verify_time_plan(B: int, Hq: int, Hkv: int, D: int, n_ctx: int, N: int, elem_bytes: int,
                     bandwidth: float, compute_shared: float, compute_tiles: float, overhead: float) -> float:
    """T_verify(N) following the kernel plan (BASTION's latency model,
    calibrated on measured runs, with the structure of the kernels that run):

        T = max(KV / bandwidth, Q * F_pad / compute_k) + W / bandwidth + overhead

    KV = 2 B Hkv n_ctx D e (the context rows, read once); F_pad = 4 B Hkv
    tiles rows n_ctx D (the MFMA work of every row of every row tile, padding
    included); compute_k = compute_shared for the shared-tile kernel, else
    compute_tiles; Q = ceil(Wg / 256) * 256 / Wg, the rounds in which the
    Wg = B Hkv tiles splits context workgroups run on 256 CUs (one workgroup
    per CU) over the rounds a perfectly divided grid would need; W =
    2 B Hq N parts (D + 1) 4 (the float32 partial rows and their
    log-sum-exps, written by the partial kernel and read by the merge).  The
    constants are effective ones: the fit lets them absorb what the terms
    leave out (fixed per-call costs, L2 reuse)."""
    shared, rows, tiles, splits, parts = kernel_plan(B, Hq, Hkv, n_ctx, N, elem_bytes)
    kv = 2.0 * B * Hkv * n_ctx * D * elem_bytes
    f_pad = 4.0 * B * Hkv * tiles * rows * n_ctx * D
    groups = B * Hkv * tiles * splits
    q = (-(-groups // 256)) * 256.0 / groups if groups > 0 else 1.0
    w = 2.0 * B * Hq * N * parts * (D + 1) * 4
    comp = compute_shared if shared else compute_tiles
    return max(kv / bandwidth, q * f_pad / comp) + w / bandwidth + overhead


def choose_tree_size(a_hat_cum: Sequence[float], t_verify: Sequence[float], t_draft: float, l_ar: float):
    """Tree size from the stopping rule: a_hat_cum[n - 1] is the surrogate
    A_hat of the best-first tree of n nodes, t_verify[n - 1] the estimated
    T_verify(n).  Returns (N, S) with S[n - 1] = A_hat(n) * L_AR / C(n),
    C(n) = t_draft + t_verify(n), and N the first n whose successor does not
    improve S (or the largest n)."""
    a = np.asarray(a_hat_cum, dtype=np.float64)
    t = np.asarray(t_verify, dtype=np.float64)
    S = a * l_ar / (t_draft + t)
    n = 1
    while n < S.size and S[n] > S[n - 1]:
        n += 1
    return n, S
