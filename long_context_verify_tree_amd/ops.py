"""Thin Python binding over libverify_attn.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/verify_attn.h``; this module turns torch tensors into pointers,
strides and the current HIP stream, allocates outputs and workspaces with
torch, and raises ``VerifyAttnError`` on a non-zero status.  There is no
fallback: if the library cannot be loaded, every call raises.

Names follow the C ABI: ``verify_attn_dense``, ``verify_attn_sparse``,
``select_verify_set`` (plus the two stages ``verify_attn_partials`` /
``verify_attn_merge`` and the workspace-size queries).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch  # noqa: F401  -- must be loaded first so the library binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libverify_attn.so")

VA_OK, VA_EINVAL, VA_EUNSUPPORTED, VA_EWORKSPACE, VA_EHIP = range(5)
VA_FP32, VA_BF16 = 0, 1


class VerifyAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"verify_attn status {status}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("L", ctypes.c_int32), ("N", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 3), ("kc_stride", ctypes.c_int64 * 3),
        ("vc_stride", ctypes.c_int64 * 3), ("kd_stride", ctypes.c_int64 * 3),
        ("vd_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
    ]


_lib = None
_P = ctypes.c_void_p
_DESC_P = ctypes.POINTER(AttnDesc)


def _declare(lib):
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "va_attn_workspace_size": (i32, [_DESC_P, i32, ctypes.POINTER(sz)]),
        "verify_attn_dense": (i32, [_DESC_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "verify_attn_sparse": (i32, [_DESC_P, _P, _P, _P, _P, _P, _P, _P, i32, i64, _P, _P, _P, sz, _P]),
        "verify_attn_partials": (i32, [_DESC_P, _P, _P, _P, _P, _P, _P, _P, i32, i64, _P, sz, _P]),
        "verify_attn_merge": (i32, [_DESC_P, i32, _P, _P, _P, sz, _P]),
        "verify_attn_dense_noalloc": (i32, [_DESC_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "va_noalloc_scratch_bytes": (sz, []),
        "va_select_workspace_size": (i32, [i32, i32, ctypes.POINTER(sz)]),
        "select_verify_set": (i32, [_P, _P, i32, i32, i64, i32, i32, i32, i32, _P, _P, sz, _P]),
        "accept_commit": (i32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "va_scores_workspace_size": (i32, [_P, _P]),
        "build_draft_tree": (i32, [_P, _P, i32, i32, i32, i32, _P, _P, _P, _P, _P]),
        "va_verify_time_model": (i32, [_P, i32, _P, i32, _P]),
        "va_choose_tree_size": (i32, [_P, _P, i32, ctypes.c_double, ctypes.c_double, _P]),
        "importance_scores": (i32, [_P, _P, _P, _P, i64, _P, sz, _P]),
        "verify_set_recovery": (i32, [_P, i64, i32, i32, _P, i32, i64, i32, i32, _P, _P]),
        "va_status_str": (ctypes.c_char_p, [i32]),
        "va_last_error": (ctypes.c_char_p, []),
        "va_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def load(path: Optional[str] = None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m long_context_verify_tree_amd.build`")
        lib = ctypes.CDLL(p)
        _declare(lib)
        _lib = lib
    return _lib


def _check(status: int):
    if status != VA_OK:
        raise VerifyAttnError(status, _lib.va_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return VA_BF16
    if t.dtype == torch.float32:
        return VA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _row_stride(t: torch.Tensor, row_len: int) -> int:
    """Row stride of a [B, n] tensor; a single row may carry any stride (a
    broadcast view has 0), and its length stands in for it."""
    return t.stride(0) if t.shape[0] > 1 else row_len


def _strides3(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("tensors must be 4-D with a unit innermost stride")
    return (ctypes.c_int64 * 3)(*[t.stride(a) for a in range(3)])


def make_desc(q, k_cache, v_cache, k_draft, v_draft, out, scale: Optional[float] = None) -> AttnDesc:
    B, Hq, N, D = q.shape
    Hkv = k_draft.shape[1]
    L = k_cache.shape[2] if k_cache is not None else 0
    d = AttnDesc()
    d.B, d.Hq, d.Hkv, d.D, d.L, d.N = B, Hq, Hkv, D, L, N
    d.dtype = _dtype_code(q)
    d.scale = 0.0 if scale is None else float(scale)
    d.q_stride = _strides3(q)
    zero = (ctypes.c_int64 * 3)(0, 0, 0)
    d.kc_stride = _strides3(k_cache) if k_cache is not None else zero
    d.vc_stride = _strides3(v_cache) if v_cache is not None else zero
    d.kd_stride = _strides3(k_draft)
    d.vd_stride = _strides3(v_draft)
    d.o_stride = _strides3(out)
    return d


def _check_inputs(q, k_cache, v_cache, k_draft, v_draft, parent):
    ts = [t for t in (q, k_cache, v_cache, k_draft, v_draft) if t is not None]
    dev = q.device
    for t in ts:
        if t.device != dev or t.dtype != q.dtype:
            raise ValueError("q, caches and drafts must share device and dtype")
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    B, Hq, N, D = q.shape
    Hkv = k_draft.shape[1]
    if k_draft.shape != (B, Hkv, N, D) or v_draft.shape != (B, Hkv, N, D):
        raise ValueError("k_draft / v_draft must be [B, Hkv, N, D]")
    if k_cache is not None and (k_cache.shape[:2] != (B, Hkv) or k_cache.shape[3] != D
                                or v_cache.shape != k_cache.shape):
        raise ValueError("k_cache / v_cache must be [B, Hkv, L, D]")
    if parent.shape != (B, N) or parent.dtype != torch.int32 or not parent.is_contiguous():
        raise ValueError("parent must be a contiguous int32 [B, N] tensor")


def workspace_size(desc: AttnDesc, n_ctx: int) -> int:
    load()
    n = ctypes.c_size_t()
    _check(_lib.va_attn_workspace_size(ctypes.byref(desc), n_ctx, ctypes.byref(n)))
    return n.value


def _workspace(desc, n_ctx, device, workspace):
    need = workspace_size(desc, n_ctx)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace


def _outputs(q, out, lse, want_lse):
    B, Hq, N, D = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    return out, lse


def verify_attn_dense(q, k_cache, v_cache, k_draft, v_draft, parent, *, out=None, lse=None,
                      scale: Optional[float] = None, workspace=None,
                      want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense verification attention; returns (out [B,Hq,N,D], lse [B,Hq,N] or None)."""
    load()
    _check_inputs(q, k_cache, v_cache, k_draft, v_draft, parent)
    out, lse = _outputs(q, out, lse, want_lse)
    desc = make_desc(q, k_cache, v_cache, k_draft, v_draft, out, scale)
    ws = _workspace(desc, desc.L, q.device, workspace)
    _check(_lib.verify_attn_dense(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft),
                                  _ptr(v_draft), _ptr(parent), _ptr(out), _ptr(lse), _ptr(ws),
                                  ws.numel(), _stream(q.device)))
    return out, lse


def verify_attn_dense_noalloc(q, k_cache, v_cache, k_draft, v_draft, parent, *, out=None, lse=None,
                              scale: Optional[float] = None,
                              want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense verification through the library's fixed device scratch (no
    workspace; the library allocates nothing).  Calls on one GPU share that
    scratch and must not overlap in time."""
    load()
    _check_inputs(q, k_cache, v_cache, k_draft, v_draft, parent)
    out, lse = _outputs(q, out, lse, want_lse)
    desc = make_desc(q, k_cache, v_cache, k_draft, v_draft, out, scale)
    _check(_lib.verify_attn_dense_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft),
                                          _ptr(v_draft), _ptr(parent), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def noalloc_scratch_bytes() -> int:
    load()
    return int(_lib.va_noalloc_scratch_bytes())


def verify_attn_sparse(q, k_cache, v_cache, k_draft, v_draft, parent, verify_idx, *, out=None, lse=None,
                       scale: Optional[float] = None, workspace=None,
                       want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse verification over verify_idx [B, K] int32; returns (out, lse)."""
    load()
    _check_inputs(q, k_cache, v_cache, k_draft, v_draft, parent)
    if verify_idx.dtype != torch.int32 or verify_idx.dim() != 2 or \
            (verify_idx.shape[1] > 1 and verify_idx.stride(1) != 1):
        raise ValueError("verify_idx must be int32 [B, K] with unit column stride")
    K = verify_idx.shape[1]
    out, lse = _outputs(q, out, lse, want_lse)
    desc = make_desc(q, k_cache, v_cache, k_draft, v_draft, out, scale)
    ws = _workspace(desc, K, q.device, workspace)
    _check(_lib.verify_attn_sparse(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft),
                                   _ptr(v_draft), _ptr(parent), _ptr(verify_idx), K,
                                   _row_stride(verify_idx, K) if K else 0, _ptr(out), _ptr(lse), _ptr(ws),
                                   ws.numel(), _stream(q.device)))
    return out, lse


def verify_attn_partials(desc: AttnDesc, q, k_cache, v_cache, k_draft, v_draft, parent, workspace,
                         verify_idx=None):
    """First stage only (split partials + tree partial) into ``workspace``."""
    load()
    if verify_idx is not None and (verify_idx.dtype != torch.int32 or verify_idx.dim() != 2 or
                                   (verify_idx.shape[1] > 1 and verify_idx.stride(1) != 1)):
        raise ValueError("verify_idx must be int32 [B, K] with unit column stride")
    K = verify_idx.shape[1] if verify_idx is not None else desc.L
    stride = _row_stride(verify_idx, K) if verify_idx is not None else 0
    # the library tells a sparse call by a non-NULL index pointer; an empty
    # [B, 0] list may have none, and with K = 0 no index is read
    idx_ptr = None
    if verify_idx is not None:
        idx_ptr = _ptr(verify_idx) if verify_idx.numel() > 0 else _ptr(workspace)
    _check(_lib.verify_attn_partials(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft),
                                     _ptr(v_draft), _ptr(parent), idx_ptr, K, stride, _ptr(workspace),
                                     workspace.numel(), _stream(q.device)))


def verify_attn_merge(desc: AttnDesc, n_ctx: int, out, lse, workspace):
    """Second stage only: log-sum-exp merge of the partials in ``workspace``."""
    load()
    _check(_lib.verify_attn_merge(ctypes.byref(desc), n_ctx, _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream(out.device)))


def select_workspace_size(B: int, L: int) -> int:
    load()
    n = ctypes.c_size_t()
    _check(_lib.va_select_workspace_size(B, L, ctypes.byref(n)))
    return n.value


def select_verify_set(draft_score, target_score, *, sink: int, window: int, top_m: int, budget: int,
                      out=None, workspace=None) -> torch.Tensor:
    """I_verify per sequence: int32 [B, min(budget, L)], ascending."""
    load()
    if draft_score.shape != target_score.shape or draft_score.dim() != 2:
        raise ValueError("scores must both be [B, L]")
    if draft_score.dtype != torch.float32 or target_score.dtype != torch.float32:
        raise ValueError("scores must be float32")
    B, L = draft_score.shape
    if draft_score.stride(1) != 1 or target_score.stride(1) != 1 or \
            _row_stride(draft_score, L) != _row_stride(target_score, L):
        raise ValueError("score rows must be contiguous with a common row stride")
    k_out = min(budget, L)
    if out is None:
        out = torch.empty((B, k_out), dtype=torch.int32, device=draft_score.device)
    need = select_workspace_size(B, L)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=draft_score.device)
    _check(_lib.select_verify_set(_ptr(draft_score), _ptr(target_score), B, L, _row_stride(draft_score, L) if B else L,
                                  sink, window, top_m, budget, _ptr(out), _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0,
                                  _stream(draft_score.device)))
    return out


class ScoreDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hs", ctypes.c_int32), ("M", ctypes.c_int32), ("D", ctypes.c_int32),
                ("L", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3)]


def make_score_desc(q, k, scale: Optional[float] = None) -> ScoreDesc:
    """q [B, Hs, M, D], k [B, Hs, L, D] (bf16, unit innermost stride)."""
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise ValueError("importance scores take bf16 q and k")
    B, Hs, M, D = q.shape
    if k.shape[:2] != (B, Hs) or k.shape[3] != D:
        raise ValueError("k must be [B, Hs, L, D]")
    d = ScoreDesc()
    d.B, d.Hs, d.M, d.D, d.L, d.dtype = B, Hs, M, D, k.shape[2], VA_BF16
    d.scale = 0.0 if scale is None else float(scale)
    d.q_stride = _strides3(q)
    d.k_stride = _strides3(k)
    return d


def scores_workspace_size(desc: ScoreDesc) -> int:
    load()
    n = ctypes.c_size_t()
    _check(_lib.va_scores_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def importance_scores(q, k, scale: Optional[float] = None, out=None, workspace=None,
                      desc: Optional[ScoreDesc] = None) -> torch.Tensor:
    """Global importance map [B, L] float32 from the scoring heads' q and k."""
    load()
    if desc is None:
        desc = make_score_desc(q, k, scale)
    if out is None:
        out = torch.empty(desc.B, desc.L, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or out.stride(1) != 1:
        raise ValueError("out must be float32 with contiguous rows")
    if workspace is None:
        workspace = torch.empty(scores_workspace_size(desc), dtype=torch.uint8, device=q.device)
    _check(_lib.importance_scores(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(out), _row_stride(out, desc.L),
                                  _ptr(workspace),
                                  workspace.numel(), _stream(q.device)))
    return out


def verify_set_recovery(score, verify_idx, rows: int, out=None, accumulate: bool = False) -> torch.Tensor:
    """Attention Recovery Rate [B] float32 of the verify sets verify_idx
    [B, K] from (a piece of) the importance map score [B, L] of all `rows`
    verification query rows; accumulate adds the piece's share to out."""
    load()
    if score.dtype != torch.float32 or score.dim() != 2 or score.stride(1) != 1:
        raise ValueError("score must be float32 [B, L] with contiguous rows")
    if verify_idx.dtype != torch.int32 or verify_idx.dim() != 2 or \
            (verify_idx.shape[1] > 1 and verify_idx.stride(1) != 1):
        raise ValueError("verify_idx must be int32 [B, K] with unit column stride")
    B, L = score.shape
    K = verify_idx.shape[1]
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs out")
        out = torch.empty(B, dtype=torch.float32, device=score.device)
    _check(_lib.verify_set_recovery(_ptr(score), _row_stride(score, L), B, L, _ptr(verify_idx), K,
                                    _row_stride(verify_idx, K) if K else 0, rows, int(accumulate), _ptr(out),
                                    _stream(score.device)))
    return out


def attention_recovery(q, k_cache, verify_idx, workspace=None) -> torch.Tensor:
    """Attention Recovery Rate [B] of verify_idx for the verification rows q
    [B, Hq, N, D] over k_cache [B, Hkv, L, D]: importance_scores over every
    query row (the G query heads of a KV head are its G * N rows, taken 32 at
    a time), each piece's share accumulated by verify_set_recovery."""
    B, Hq, N, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    L = k_cache.shape[2]
    rows = q.reshape(B, Hkv, G * N, D)
    score = torch.empty(B, L, dtype=torch.float32, device=q.device)
    arr = torch.empty(B, dtype=torch.float32, device=q.device)
    first = True
    for kvh in range(Hkv):
        for r0 in range(0, G * N, 32):
            importance_scores(rows[:, kvh:kvh + 1, r0:r0 + 32], k_cache[:, kvh:kvh + 1], out=score,
                              workspace=workspace)
            verify_set_recovery(score, verify_idx, Hq * N, out=arr, accumulate=not first)
            first = False
    return arr


def make_commit_desc(k_cache, v_cache, k_draft, v_draft) -> AttnDesc:
    """Descriptor for accept_commit: caches [B, Hkv, capacity, D], drafts
    [B, Hkv, N, D] (desc.L = capacity; query/output fields unused)."""
    if k_cache.dtype != k_draft.dtype or v_cache.dtype != k_draft.dtype or v_draft.dtype != k_draft.dtype:
        raise ValueError("caches and drafts must share a dtype")
    B, Hkv, N, D = k_draft.shape
    if k_cache.shape[:2] != (B, Hkv) or k_cache.shape[3] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [B, Hkv, capacity, D]")
    d = AttnDesc()
    d.B, d.Hq, d.Hkv, d.D, d.L, d.N = B, Hkv, Hkv, D, k_cache.shape[2], N
    d.dtype = _dtype_code(k_cache)
    d.scale = 0.0
    zero = (ctypes.c_int64 * 3)(0, 0, 0)
    d.q_stride = zero
    d.o_stride = zero
    d.kc_stride = _strides3(k_cache)
    d.vc_stride = _strides3(v_cache)
    d.kd_stride = _strides3(k_draft)
    d.vd_stride = _strides3(v_draft)
    return d


def accept_commit(k_cache, v_cache, k_draft, v_draft, parent, accepted, cache_len, new_len=None,
                  desc: Optional[AttnDesc] = None) -> torch.Tensor:
    """Append each sequence's accepted draft path to its cache in place.

    k_cache/v_cache [B, Hkv, capacity, D]; accepted/cache_len int32 [B].
    Returns new_len int32 [B] (cache_len + path length).  `desc` (from
    make_commit_desc for the same tensors) skips rebuilding the descriptor."""
    load()
    if desc is None:
        desc = make_commit_desc(k_cache, v_cache, k_draft, v_draft)
        B, N = desc.B, desc.N
        for t, name in ((parent, "parent"), (accepted, "accepted"), (cache_len, "cache_len")):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous int32")
        if parent.shape != (B, N) or accepted.shape != (B,) or cache_len.shape != (B,):
            raise ValueError("parent [B, N], accepted [B] and cache_len [B] expected")
    if new_len is None:
        new_len = torch.empty(desc.B, dtype=torch.int32, device=k_cache.device)
    for t, name in ((cache_len, "cache_len"), (accepted, "accepted"), (parent, "parent")):
        lo, hi = t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()
        if new_len.data_ptr() < hi and lo < new_len.data_ptr() + new_len.numel() * 4:
            raise ValueError(f"new_len must not overlap {name} (the library rejects in-place length updates)")
    _check(_lib.accept_commit(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k_draft), _ptr(v_draft),
                              _ptr(parent), _ptr(accepted), _ptr(cache_len), _ptr(new_len), _stream(k_cache.device)))
    return new_len


def build_draft_tree(cand_prob, cand_token, N: int):
    """Best-first draft tree of N nodes per sequence from candidates
    cand_prob float32 [B, K, T] and cand_token int32 [B, K, T].
    Returns (parent int32 [B, N], token int32 [B, N], rho float32 [B, N],
    a_hat float32 [B])."""
    load()
    if cand_prob.dtype != torch.float32 or cand_token.dtype != torch.int32:
        raise ValueError("cand_prob must be float32 and cand_token int32")
    if cand_prob.dim() != 3 or cand_token.shape != cand_prob.shape:
        raise ValueError("cand_prob and cand_token must both be [B, K, T]")
    if not (cand_prob.is_contiguous() and cand_token.is_contiguous()):
        raise ValueError("candidates must be contiguous")
    B, K, T = cand_prob.shape
    dev = cand_prob.device
    parent = torch.empty(B, N, dtype=torch.int32, device=dev)
    token = torch.empty(B, N, dtype=torch.int32, device=dev)
    rho = torch.empty(B, N, dtype=torch.float32, device=dev)
    a_hat = torch.empty(B, dtype=torch.float32, device=dev)
    _check(_lib.build_draft_tree(_ptr(cand_prob), _ptr(cand_token), B, K, T, N, _ptr(parent), _ptr(token), _ptr(rho),
                                 _ptr(a_hat), _stream(dev)))
    return parent, token, rho, a_hat


class TimeConsts(ctypes.Structure):
    _fields_ = [("bandwidth", ctypes.c_double), ("compute_shared", ctypes.c_double),
                ("compute_tiles", ctypes.c_double), ("overhead", ctypes.c_double)]


def verify_time_model(desc: AttnDesc, n_ctx: int, bandwidth: float, compute_shared: float, compute_tiles: float,
                      overhead: float, N: int) -> float:
    """Estimated verification time (seconds) of N draft nodes, following the
    library's kernel plan, with calibrated constants."""
    load()
    k = TimeConsts(bandwidth, compute_shared, compute_tiles, overhead)
    out = ctypes.c_double()
    _check(_lib.va_verify_time_model(ctypes.byref(desc), n_ctx, ctypes.byref(k), N, ctypes.byref(out)))
    return out.value


def choose_tree_size(a_hat_cum, t_verify, t_draft: float, l_ar: float) -> int:
    """Tree size from the stop-at-first-decrease rule (host arrays)."""
    load()
    a = np.ascontiguousarray(np.asarray(a_hat_cum, dtype=np.float32))
    t = np.ascontiguousarray(np.asarray(t_verify, dtype=np.float64))
    if a.shape != t.shape or a.ndim != 1:
        raise ValueError("a_hat_cum and t_verify must be 1-D of equal length")
    n = ctypes.c_int32()
    _check(_lib.va_choose_tree_size(a.ctypes.data_as(ctypes.c_void_p), t.ctypes.data_as(ctypes.c_void_p), a.size,
                                    t_draft, l_ar, ctypes.byref(n)))
    return n.value
