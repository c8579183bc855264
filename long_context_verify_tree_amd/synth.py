"""Seeded synthetic inputs for speculative-verification attention.

This module only draws random numbers and lays them out; it performs none of
the method's arithmetic.  Both the HIP path (tests, bench) and the CPU oracle
read inputs produced here, so the two sides always see identical bits.

Workload shapes follow the long-context speculative-decoding setting of the
Dustin summary ("Definizione del Problema": 32k-token contexts, multi-batch)
and the tree verification of LongSpec ("Tree Attention Ibrida") and BASTION
("Drafting a Diffusione a Blocchi Basato su Albero": a prefix tree of draft
candidates, carried here as a parent array).  The pages use PG-19, LongBench
and similar suites; seeded synthetic tensors of the same shapes stand in for
them.

Recipe (one ``numpy.random.Generator(PCG64)`` per tensor, children of
``SeedSequence(seed).spawn(8)`` in the fixed order q, k_cache, v_cache,
k_draft, v_draft, tree, draft_score, target_score):

* q, K/V cache, draft K/V: N(0, 1) drawn as float32 in chunks, then rounded
  to bfloat16 with round-to-nearest-even (float32 configs keep the float32).
* tree: chain (``parent[i] = i - 1``), uniform (``parent[i] ~ U[-1, i-1]``)
  or a random prefix tree with bounded depth and branching, drawn per
  sequence.
* scores: LogNormal(0, 2) float32, one row of L per sequence.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
FP32 = "fp32"

_CHUNK = 1 << 24  # elements drawn per chunk; fixes the stream layout


@dataclasses.dataclass(frozen=True)
class VerifyConfig:
    """Shape of one verification problem (one target-model layer)."""

    name: str
    B: int            # sequences in the batch
    Hq: int           # query heads
    Hkv: int          # key/value heads (GQA groups of Hq // Hkv query heads)
    D: int            # head dimension
    L: int            # committed context length (KV cache rows)
    N: int            # draft nodes per sequence
    tree: str         # "chain" | "uniform" | "prefix"
    dtype: str        # BF16 | FP32
    seed: int
    max_depth: int = 0        # prefix trees: depth bound (root children have depth 1)
    max_branch: int = 0       # prefix trees: children per node (and per root) bound
    sparse: bool = False      # verify over a selected subset I_verify
    dense: bool = True        # verify over the whole cache
    sink: int = 0
    window: int = 0
    top_m: int = 0
    budget: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "VerifyConfig":
        return dataclasses.replace(self, **kw)


# The five workloads, smallest first.
CONFIGS = {
    "tiny_fp32": VerifyConfig(
        "tiny_fp32", B=1, Hq=4, Hkv=1, D=64, L=256, N=8, tree="uniform",
        dtype=FP32, seed=101),
    "llama3_8b_chain8_L32k": VerifyConfig(
        "llama3_8b_chain8_L32k", B=8, Hq=32, Hkv=8, D=128, L=32768, N=8,
        tree="chain", dtype=BF16, seed=202),
    "llama3_8b_tree64_L64k": VerifyConfig(
        "llama3_8b_tree64_L64k", B=4, Hq=32, Hkv=8, D=128, L=65536, N=64,
        tree="prefix", max_depth=8, max_branch=4, dtype=BF16, seed=303),
    "qwen25_7b_sparse2048_L32k": VerifyConfig(
        "qwen25_7b_sparse2048_L32k", B=16, Hq=28, Hkv=4, D=128, L=32768, N=8,
        tree="chain", dtype=BF16, seed=404, sparse=True, dense=False,
        sink=4, window=256, top_m=1024, budget=2048),
    "l70b_tree128_L128k": VerifyConfig(
        "l70b_tree128_L128k", B=4, Hq=64, Hkv=8, D=128, L=131072, N=128,
        tree="prefix", max_depth=12, max_branch=4, dtype=BF16, seed=505,
        sparse=True, dense=True, sink=4, window=256, top_m=2048, budget=4096),
}
CONFIG_ORDER = list(CONFIGS)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, _CHUNK):
        c = flat_u[s:s + _CHUNK].astype(np.uint64)
        c = (c + 0x7FFF + ((c >> 16) & 1)) >> 16
        flat_o[s:s + _CHUNK] = c.astype(np.uint16)
    return out


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == FP32:
        out = np.empty(n, dtype=np.float32)
        for s in range(0, n, _CHUNK):
            out[s:s + _CHUNK] = rng.standard_normal(min(_CHUNK, n - s), dtype=np.float32)
        return out.reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        out[s:s + _CHUNK] = f32_to_bf16_bits(
            rng.standard_normal(min(_CHUNK, n - s), dtype=np.float32))
    return out.reshape(shape)


def chain_parents(N: int) -> np.ndarray:
    return np.arange(-1, N - 1, dtype=np.int32)


def uniform_parents(rng: np.random.Generator, N: int) -> np.ndarray:
    """parent[i] uniform over [-1, i-1] (always topologically ordered)."""
    return np.array([rng.integers(-1, i) if i > 0 else -1 for i in range(N)],
                    dtype=np.int32)


def prefix_tree_parents(rng: np.random.Generator, N: int, max_depth: int,
                        max_branch: int) -> np.ndarray:
    """Random prefix tree in topological order with depth and branching bounds.

    Node i picks its parent uniformly among the virtual root (-1, while it
    has fewer than ``max_branch`` children) and the earlier nodes whose depth
    is below ``max_depth`` and that have fewer than ``max_branch`` children.
    """
    parent = np.empty(N, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int64)
    children = np.zeros(N, dtype=np.int64)
    root_children = 0
    for i in range(N):
        cand = [-1] if root_children < max_branch else []
        cand += [j for j in range(i) if depth[j] < max_depth and children[j] < max_branch]
        if not cand:
            raise ValueError("tree bounds too tight for N nodes")
        p = cand[int(rng.integers(len(cand)))]
        parent[i] = p
        if p < 0:
            root_children += 1
            depth[i] = 1
        else:
            children[p] += 1
            depth[i] = depth[p] + 1
    return parent


@dataclasses.dataclass
class VerifyInputs:
    cfg: VerifyConfig
    q: np.ndarray          # [B, Hq, N, D]   uint16 bf16 bits or float32
    k_cache: np.ndarray    # [B, Hkv, L, D]
    v_cache: np.ndarray    # [B, Hkv, L, D]
    k_draft: np.ndarray    # [B, Hkv, N, D]
    v_draft: np.ndarray    # [B, Hkv, N, D]
    parent: np.ndarray     # [B, N] int32
    draft_score: Optional[np.ndarray]   # [B, L] float32 (sparse configs)
    target_score: Optional[np.ndarray]  # [B, L] float32


def make_parents(cfg: VerifyConfig, rng: np.random.Generator) -> np.ndarray:
    rows = []
    for _ in range(cfg.B):
        if cfg.tree == "chain":
            rows.append(chain_parents(cfg.N))
        elif cfg.tree == "uniform":
            rows.append(uniform_parents(rng, cfg.N))
        elif cfg.tree == "prefix":
            rows.append(prefix_tree_parents(rng, cfg.N, cfg.max_depth, cfg.max_branch))
        elif cfg.tree == "star":
            rows.append(np.full(cfg.N, -1, dtype=np.int32))
        else:
            raise ValueError(cfg.tree)
    return np.stack(rows).astype(np.int32)


def make_scores(rng: np.random.Generator, B: int, L: int) -> np.ndarray:
    return rng.lognormal(0.0, 2.0, size=(B, L)).astype(np.float32)


def make_inputs(cfg: VerifyConfig, scores: Optional[bool] = None) -> VerifyInputs:
    """Draw every input tensor of ``cfg`` from its seed."""
    ss = np.random.SeedSequence(cfg.seed).spawn(8)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    B, Hq, Hkv, D, L, N = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.L, cfg.N
    q = _normal(g[0], (B, Hq, N, D), cfg.dtype)
    kc = _normal(g[1], (B, Hkv, L, D), cfg.dtype)
    vc = _normal(g[2], (B, Hkv, L, D), cfg.dtype)
    kd = _normal(g[3], (B, Hkv, N, D), cfg.dtype)
    vd = _normal(g[4], (B, Hkv, N, D), cfg.dtype)
    parent = make_parents(cfg, g[5])
    want_scores = cfg.sparse if scores is None else scores
    ds = make_scores(g[6], B, L) if want_scores else None
    ts = make_scores(g[7], B, L) if want_scores else None
    return VerifyInputs(cfg, q, kc, vc, kd, vd, parent, ds, ts)


def small_variant(cfg: VerifyConfig, L: int, B: Optional[int] = None,
                  seed_offset: int = 7) -> VerifyConfig:
    """The same head shape and tree kind at a reduced context length."""
    kw = dict(L=L, seed=cfg.seed + seed_offset)
    if B is not None:
        kw["B"] = B
    if cfg.sparse:
        kw["budget"] = min(cfg.budget, max(cfg.sink + cfg.window, L // 4))
        kw["window"] = min(cfg.window, max(L // 8, 0))
        kw["top_m"] = min(cfg.top_m, max(kw["budget"] // 2, 0))
        kw["budget"] = max(kw["budget"], cfg.sink + kw["window"])
    return cfg.with_(name=f"{cfg.name}@L{L}", **kw)
