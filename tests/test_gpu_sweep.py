"""Seeded sweep of random shapes through the C ABI against the oracle.

Each case draws a problem shape (dtype, head dimension, batch, GQA group,
draft nodes, tree shape, context length, cache layout (head-major, or
token-major passed as strided views), and for sparse cases a verify set of
random size and order) from a fixed seed, so the list is the same on
every run; together they reach combinations of plan branches (which partial
kernel, row tiles, ragged last tiles, one or many context splits, the tree
alone, the tree in the last split) that the hand-picked cases do not.  The
sizes are bounded (about 1e9 multiply-adds per case) so that the fp64
oracle takes a few seconds at most for any case and about 20 s for all.  Expected values come only from ``oracle`` (LongSpec, "Tree Attention
Ibrida": the tree-masked attention over context and drafts; Dustin,
"Aggregazione Ibrida dell'Attenzione": the context restricted to the verify
set)."""

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo
from long_context_verify_tree_amd import synth
from _util import check_rows, device_inputs, out_to_f64

pytestmark = pytest.mark.gpu

N_CASES = 96


def say(*a):
    print(*a, flush=True)


def draw_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    while len(cases) < N_CASES:
        dtype = synth.BF16 if rng.random() < 0.75 else synth.FP32
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 7, 8]))
        N = int(rng.choice([1, 3, 8, 17, 33, 64, 65, 100, 128, 256]))
        B = int(rng.choice([1, 2, 3, 4]))
        L = int(rng.choice([0, 1, 7, 31, 100, 511, 513, 1500, 5000, 20000, 40000]))
        tree = str(rng.choice(["chain", "uniform", "star"]))
        sparse = L > 0 and rng.random() < 0.4
        K = int(rng.integers(0, L + 1)) if sparse else None
        n_ctx = K if sparse else L
        # keep the fp64 oracle to about 1e9 multiply-adds per case
        if B * G * Hkv * N * (n_ctx + N) * D > 1e9:
            continue
        tokmajor = L > 0 and rng.random() < 0.2   # caches stored token-major, passed as strided views
        cases.append(dict(dtype=dtype, D=D, Hkv=Hkv, G=G, N=N, B=B, L=L, tree=tree, K=K, tokmajor=tokmajor,
                          seed=int(rng.integers(1 << 30))))
    return cases


# and two the draw leaves out: the gathered shared-tile kernel over several
# context splits (the tree walked by the last one)
CASES = draw_cases() + [
    dict(dtype=synth.BF16, D=128, Hkv=2, G=8, N=33, B=2, L=20000, tree="uniform", K=9000, tokmajor=False,
         seed=77001),
    dict(dtype=synth.BF16, D=64, Hkv=1, G=4, N=64, B=1, L=20000, tree="chain", K=15000, tokmajor=False,
         seed=77002),
]


def case_id(c):
    mode = f"sparse{c['K']}" if c["K"] is not None else "dense"
    tm = "_tokmajor" if c["tokmajor"] else ""
    return f"{c['dtype']}_D{c['D']}_B{c['B']}_G{c['G']}x{c['Hkv']}_N{c['N']}_{c['tree']}_L{c['L']}_{mode}{tm}"


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_random_shape_matches_oracle(gpu_lib, case):
    c = case
    cfg = synth.VerifyConfig("sweep", B=c["B"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"], L=c["L"], N=c["N"],
                             tree=c["tree"], dtype=c["dtype"], seed=c["seed"])
    x = synth.make_inputs(cfg)
    n_ctx = c["K"] if c["K"] is not None else c["L"]
    es = 2 if c["dtype"] == synth.BF16 else 4
    plan = vo.kernel_plan(cfg.B, cfg.Hq, cfg.Hkv, n_ctx, cfg.N, es, sparse=c["K"] is not None)
    say(f"case sweep {case_id(c)}: shared-tile kernel {plan[0]}, row tiles {plan[2]}, splits {plan[3]}, "
        f"parts {plan[4]}")
    d = device_inputs(x)
    if c["tokmajor"]:
        d["k_cache"] = d["k_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        d["v_cache"] = d["v_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if c["K"] is None:
        out, lse = gpu_lib.verify_attn_dense(**d)
        ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    else:
        rng = np.random.default_rng(c["seed"])
        idx = np.stack([rng.permutation(cfg.L)[:c["K"]] for _ in range(cfg.B)]).astype(np.int32)
        if rng.random() < 0.5:
            idx = np.sort(idx, axis=1)
        out, lse = gpu_lib.verify_attn_sparse(**d, verify_idx=torch.from_numpy(idx).cuda())
        ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
    torch.cuda.synchronize()
    check_rows(out_to_f64(out), ref, lse.cpu().numpy().astype(np.float64), rlse, cfg.dtype, case_id(c))
