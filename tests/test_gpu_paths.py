"""GPU parity of every kernel variant and plan branch the C ABI can reach.

Each case names the path it forces (which partial kernel instance, how many
parts the merge joins), checks through the ABI against the CPU oracle on
every output row, and prints its name before it touches the GPU.  Expected
values come only from ``oracle``.
"""

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo
from long_context_verify_tree_amd import synth
from _util import check_rows, device_inputs, out_to_f64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def cfg_of(name, **kw):
    base = dict(B=1, Hq=4, Hkv=1, D=128, L=300, N=8, tree="uniform", dtype=synth.BF16, seed=1000)
    base.update(kw)
    return synth.VerifyConfig(name, **base)


def run_dense(ops, x):
    d = device_inputs(x)
    out, lse = ops.verify_attn_dense(**d)
    torch.cuda.synchronize()
    return out_to_f64(out), lse.cpu().numpy().astype(np.float64)


def run_sparse(ops, x, idx):
    d = device_inputs(x)
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    out, lse = ops.verify_attn_sparse(**d, verify_idx=it)
    torch.cuda.synchronize()
    return out_to_f64(out), lse.cpu().numpy().astype(np.float64)


def n_parts(ops, x, n_ctx):
    """Partial slots per row of the library's workspace (the larger of the
    dense and sparse plans' part counts: context splits + the tree part),
    read back from the workspace size: rows * parts * (D + 1) floats, each
    array rounded up to 256 bytes, and a 256-byte header."""
    d = device_inputs(x)
    out = torch.empty_like(d["q"])
    desc = ops.make_desc(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], out)
    ws = ops.workspace_size(desc, n_ctx)
    rows = x.cfg.B * x.cfg.Hq * x.cfg.N
    return ws // (rows * (x.cfg.D + 1) * 4)


def test_merge_across_groups_of_parts(gpu_lib):
    # One Llama-3-8B-shape sequence at L = 32768 (32 query heads on 8 KV heads,
    # 8 chained drafts): the plan cuts the context into 32 splits, so the merge
    # joins 33 parts and rescales across its groups of 16.
    cfg = cfg_of("merge33", Hq=32, Hkv=8, L=32768, N=8, tree="chain", seed=1313)
    x = synth.make_inputs(cfg)
    parts = n_parts(gpu_lib, x, cfg.L)
    say(f"case merge across groups: {parts} parts")
    assert parts > 32
    got, glse = run_dense(gpu_lib, x)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(got, ref, glse, rlse, cfg.dtype, "merge33")


def test_merge_across_groups_peaky_late_split(gpu_lib):
    # The same plan with the dominant keys in the last splits: the running
    # maximum of the merge has to move after its first group of 16 parts.
    cfg = cfg_of("merge33late", Hq=32, Hkv=8, L=32768, N=8, tree="chain", seed=1314)
    x = synth.make_inputs(cfg)
    f = lambda a: vo.bf16_bits_to_f64(a).astype(np.float32)
    q, kc = f(x.q), f(x.k_cache)
    for kvh in range(cfg.Hkv):
        kc[0, kvh, 30000:30004] = 2.5 * q[0, kvh * 4, :4]
    x.k_cache = synth.f32_to_bf16_bits(kc)
    say("case merge across groups, dominant keys in split 29")
    got, glse = run_dense(gpu_lib, x)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(got, ref, glse, rlse, cfg.dtype, "merge33late")
    assert np.abs(ref).max() > 0.3


@pytest.mark.parametrize("D", [64, 128])
def test_dense_and_sparse_plans_on_one_workspace(gpu_lib, D):
    # bf16 with 56 query rows per KV head: a dense call runs one 64-row tile
    # per KV head (the per-wavefront kernel's bf16 two-row-block instance), a
    # sparse call two 32-row tiles, and the two plans join different part
    # counts.  Partials of either mode, each followed by a merge called on its
    # own (it reads the part count the partials wrote into the workspace
    # header), alternate on one workspace; then the one-call entry points.
    cfg = cfg_of(f"modes_D{D}", B=2, Hq=14, Hkv=2, D=D, L=5000, N=8, tree="uniform", seed=1500 + D)
    x = synth.make_inputs(cfg)
    rng = np.random.default_rng(D)
    K = 1700
    idx = np.stack([np.sort(rng.permutation(cfg.L)[:K]) for _ in range(cfg.B)]).astype(np.int32)
    pd = vo.kernel_plan(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.N, 2)
    ps = vo.kernel_plan(cfg.B, cfg.Hq, cfg.Hkv, K, cfg.N, 2, sparse=True)
    say(f"case dense/sparse plans D={D}: dense {pd}, sparse {ps}")
    assert pd[1:3] == (64, 1) and ps[1:3] == (32, 2) and pd[4] != ps[4]
    refs = {
        "dense": vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent),
        "sparse": vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx),
    }
    d = device_inputs(x)
    it = torch.from_numpy(idx).cuda()
    out = torch.empty_like(d["q"])
    lse = torch.empty(cfg.B, cfg.Hq, cfg.N, dtype=torch.float32, device="cuda")
    desc = gpu_lib.make_desc(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], out)
    ws = torch.empty(max(gpu_lib.workspace_size(desc, cfg.L), gpu_lib.workspace_size(desc, K)), dtype=torch.uint8,
                     device="cuda")
    for mode in ("sparse", "dense", "sparse", "dense"):
        say(f"case dense/sparse plans D={D}: {mode} partials, merge on its own")
        out.fill_(float("nan"))
        sp = mode == "sparse"
        gpu_lib.verify_attn_partials(desc, d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"],
                                     d["parent"], ws, verify_idx=it if sp else None)
        gpu_lib.verify_attn_merge(desc, K if sp else cfg.L, out, lse, ws)
        torch.cuda.synchronize()
        ref, rlse = refs[mode]
        check_rows(out_to_f64(out), ref, lse.cpu().numpy().astype(np.float64), rlse, cfg.dtype, f"{cfg.name}/{mode}")
    say(f"case dense/sparse plans D={D}: one-call entry points")
    got, glse = run_dense(gpu_lib, x)
    check_rows(got, *refs["dense"][:1], glse, refs["dense"][1], cfg.dtype, cfg.name + "/dense call")
    got, glse = run_sparse(gpu_lib, x, idx)
    check_rows(got, *refs["sparse"][:1], glse, refs["sparse"][1], cfg.dtype, cfg.name + "/sparse call")


@pytest.mark.parametrize("L", [0, 100, 1111])
@pytest.mark.parametrize("Hq,N", [(8, 20), (16, 20)])
def test_rows_kernel_d64(gpu_lib, L, Hq, N):
    # bf16, D = 64 and more than 64 query rows per KV head: the shared-tile
    # kernel's D = 64 instance (one and two row tiles)
    cfg = cfg_of(f"rows64_L{L}_R{Hq * N}", Hq=Hq, Hkv=1, D=64, L=L, N=N, seed=1400 + L + Hq)
    x = synth.make_inputs(cfg)
    say(f"case rows_kernel D=64 dense L={L} R={Hq * N}")
    got, glse = run_dense(gpu_lib, x)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(got, ref, glse, rlse, cfg.dtype, cfg.name)
    if L > 0:
        rng = np.random.default_rng(L)
        K = max(1, L // 3)
        idx = np.sort(rng.permutation(L)[:K]).astype(np.int32)[None]
        say(f"case rows_kernel D=64 gathered L={L} K={K}")
        got, glse = run_sparse(gpu_lib, x, idx)
        ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
        check_rows(got, ref, glse, rlse, cfg.dtype, cfg.name + "/sparse")


# gathered instances of the per-wavefront kernel: fp32 with one and two
# 32-row blocks (D 64 and 128), bf16 D = 64, and bf16 D = 128 with ragged K
GATHER_SHAPES = [
    dict(dtype=synth.FP32, D=64, Hq=4, Hkv=1, N=8),     # fp32, 32 rows: one block
    dict(dtype=synth.FP32, D=128, Hq=4, Hkv=2, N=8),    # fp32 D=128, 16 rows
    dict(dtype=synth.FP32, D=64, Hq=8, Hkv=1, N=7),     # fp32, 56 rows: two blocks
    dict(dtype=synth.FP32, D=128, Hq=6, Hkv=1, N=9),    # fp32 D=128, 54 rows: two blocks
    dict(dtype=synth.BF16, D=64, Hq=8, Hkv=2, N=5),     # bf16 D=64
    dict(dtype=synth.BF16, D=128, Hq=7, Hkv=1, N=9),    # bf16 D=128, 63 rows
]


@pytest.mark.parametrize("shape", GATHER_SHAPES, ids=lambda s: f"{s['dtype']}_D{s['D']}_R{s['Hq'] // s['Hkv'] * s['N']}")
@pytest.mark.parametrize("L,K", [(700, 233), (2100, 2100), (64, 1)])
def test_gathered_variants(gpu_lib, shape, L, K):
    cfg = cfg_of("gather", L=L, B=2, seed=1500 + L + K + shape["D"], **shape)
    x = synth.make_inputs(cfg)
    rng = np.random.default_rng(K)
    idx = np.stack([rng.permutation(L)[:K] for _ in range(cfg.B)]).astype(np.int32)
    say(f"case gathered {shape} L={L} K={K}")
    got, glse = run_sparse(gpu_lib, x, idx)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
    check_rows(got, ref, glse, rlse, cfg.dtype, f"gather {shape} L={L} K={K}")


@pytest.mark.parametrize("shape", [
    dict(dtype=synth.FP32, D=64, Hq=4, Hkv=1, N=8),
    dict(dtype=synth.BF16, D=128, Hq=8, Hkv=2, N=8),      # per-wavefront kernel
    dict(dtype=synth.BF16, D=128, Hq=16, Hkv=2, N=20),    # shared-tile kernel (160 rows)
    dict(dtype=synth.BF16, D=64, Hq=16, Hkv=1, N=9),      # shared-tile kernel, D = 64
], ids=lambda s: f"{s['dtype']}_D{s['D']}_R{s['Hq'] // s['Hkv'] * s['N']}")
def test_sparse_empty_verify_set(gpu_lib, shape):
    # K = 0: only the draft tree is attended; equals the oracle with an empty
    # context set (and dense attention over an empty cache)
    cfg = cfg_of("k0", L=500, B=2, seed=1600 + shape["D"] + shape["N"], **shape)
    x = synth.make_inputs(cfg)
    idx = np.zeros((cfg.B, 0), dtype=np.int32)
    say(f"case sparse K=0 {shape}")
    got, glse = run_sparse(gpu_lib, x, idx)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
    check_rows(got, ref, glse, rlse, cfg.dtype, f"K=0 {shape}")
    # the two stages, with an empty index list, after dense partials on the
    # same workspace
    say(f"case sparse K=0 {shape}, partials and a merge called on its own")
    d = device_inputs(x)
    out = torch.empty_like(d["q"])
    lse = torch.empty(cfg.B, cfg.Hq, cfg.N, dtype=torch.float32, device="cuda")
    desc = gpu_lib.make_desc(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], out)
    ws = torch.empty(max(gpu_lib.workspace_size(desc, cfg.L), gpu_lib.workspace_size(desc, 0)), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.verify_attn_partials(desc, d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], d["parent"], ws)
    gpu_lib.verify_attn_partials(desc, d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], d["parent"], ws,
                                 verify_idx=torch.from_numpy(idx).cuda())
    gpu_lib.verify_attn_merge(desc, 0, out, lse, ws)
    torch.cuda.synchronize()
    check_rows(out_to_f64(out), ref, lse.cpu().numpy().astype(np.float64), rlse, cfg.dtype, f"K=0 staged {shape}")
