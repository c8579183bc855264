"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case prints its name before it touches the GPU.  Inputs come from the
seeded generators in ``long_context_verify_tree_amd.synth``; expected values
come only from ``oracle``.  Small cases compare every output row; the five
workloads at full size compare sampled (sequence, head) slabs, which the
oracle computes one by one.
"""

import math

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo
from long_context_verify_tree_amd import synth
from _util import check_rows, device_inputs, out_to_f64, to_dev

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


def say(*a):
    print(*a, flush=True)


def gpu_dense(ops, x, scale=None):
    d = device_inputs(x)
    out, lse = ops.verify_attn_dense(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], d["parent"],
                                     scale=scale)
    torch.cuda.synchronize()
    return out_to_f64(out), lse.cpu().numpy().astype(np.float64)


def gpu_sparse(ops, x, idx):
    d = device_inputs(x)
    it = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    out, lse = ops.verify_attn_sparse(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], d["parent"],
                                      it)
    torch.cuda.synchronize()
    return out_to_f64(out), lse.cpu().numpy().astype(np.float64)


def oracle_all(x, idx=None, scale=None):
    return vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx,
                               scale=scale)


# ---------------------------------------------------------------------------
# small sizes: every row


def test_tiny_fp32_full(gpu_lib):
    x = synth.make_inputs(C["tiny_fp32"])
    say("case tiny_fp32 full")
    got, glse = gpu_dense(gpu_lib, x)
    ref, rlse = oracle_all(x)
    check_rows(got, ref, glse, rlse, synth.FP32, "tiny_fp32")


SMALL = [(name, L) for name in ("llama3_8b_chain8_L32k", "llama3_8b_tree64_L64k", "qwen25_7b_sparse2048_L32k",
                                "l70b_tree128_L128k") for L in (0, 16, 300, 1111)]


@pytest.mark.parametrize("name,L", SMALL)
def test_small_dense_all_rows(gpu_lib, name, L):
    cfg = synth.small_variant(C[name], L=L, B=2 if C[name].N <= 64 else 1).with_(sparse=False, dense=True)
    x = synth.make_inputs(cfg)
    say(f"case dense {cfg.name} B={cfg.B} N={cfg.N}")
    got, glse = gpu_dense(gpu_lib, x)
    ref, rlse = oracle_all(x)
    check_rows(got, ref, glse, rlse, cfg.dtype, cfg.name)


@pytest.mark.parametrize("L", [0, 77, 530])
def test_fp32_shapes(gpu_lib, L):
    # fp32 through the multi-row-tile path (G*N > 32) and D = 128
    for D, Hq, Hkv, N, tree in ((64, 8, 2, 20, "uniform"), (128, 4, 4, 9, "chain")):
        cfg = synth.VerifyConfig(f"fp32_D{D}_L{L}", B=2, Hq=Hq, Hkv=Hkv, D=D, L=L, N=N, tree=tree,
                                 dtype=synth.FP32, seed=900 + L + D)
        x = synth.make_inputs(cfg)
        say(f"case {cfg.name}")
        got, glse = gpu_dense(gpu_lib, x)
        ref, rlse = oracle_all(x)
        check_rows(got, ref, glse, rlse, synth.FP32, cfg.name)


def _observable(cfg, kind, rng):
    """Inputs whose output is dominated by a few keys (errors become visible)."""
    x = synth.make_inputs(cfg)
    f = lambda a: vo.bf16_bits_to_f64(a).astype(np.float32)
    q, kc, kd = f(x.q), f(x.k_cache), f(x.k_draft)
    G = cfg.G
    if kind == "peaky":
        q = q * 4.0
    elif kind == "needles":
        # a few context keys equal (scaled) queries of the group
        for b in range(cfg.B):
            for kvh in range(cfg.Hkv):
                pos = rng.choice(cfg.L, size=min(4, cfg.L), replace=False)
                for t, p in enumerate(pos):
                    kc[b, kvh, p] = 3.0 * q[b, kvh * G + t % G, t % cfg.N]
    elif kind == "draft_heavy":
        for b in range(cfg.B):
            for kvh in range(cfg.Hkv):
                kd[b, kvh] = 3.0 * q[b, kvh * G]
    x.q = synth.f32_to_bf16_bits(q)
    x.k_cache = synth.f32_to_bf16_bits(kc)
    x.k_draft = synth.f32_to_bf16_bits(kd)
    return x


@pytest.mark.parametrize("kind", ["peaky", "needles", "draft_heavy"])
@pytest.mark.parametrize("name", ["llama3_8b_tree64_L64k", "l70b_tree128_L128k", "qwen25_7b_sparse2048_L32k"])
def test_observability_variants(gpu_lib, name, kind):
    cfg = synth.small_variant(C[name], L=700, B=1).with_(sparse=False)
    x = _observable(cfg, kind, np.random.default_rng(7))
    say(f"case observable {kind} {cfg.name}")
    got, glse = gpu_dense(gpu_lib, x)
    ref, rlse = oracle_all(x)
    check_rows(got, ref, glse, rlse, cfg.dtype, f"{cfg.name}/{kind}")
    # the output must not be near zero in these variants
    assert np.abs(ref).max() > 0.3


def test_scale_override(gpu_lib):
    cfg = synth.small_variant(C["llama3_8b_chain8_L32k"], L=200, B=1)
    x = synth.make_inputs(cfg)
    say("case scale override")
    got, glse = gpu_dense(gpu_lib, x, scale=0.3)
    ref, rlse = oracle_all(x, scale=0.3)
    check_rows(got, ref, glse, rlse, cfg.dtype, "scale")


@pytest.mark.parametrize("shape", [
    dict(B=1, Hq=4, Hkv=4, D=128, L=100, N=1, tree="chain"),       # single node = decode, G = 1
    dict(B=2, Hq=8, Hkv=1, D=64, L=257, N=5, tree="star"),         # D = 64, wide group, star tree
    dict(B=1, Hq=2, Hkv=1, D=128, L=40, N=256, tree="chain"),      # deepest tree, 16 row tiles
    dict(B=1, Hq=6, Hkv=2, D=128, L=33, N=37, tree="uniform"),     # ragged rows and keys
    dict(B=3, Hq=4, Hkv=2, D=128, L=0, N=12, tree="uniform"),      # no context at all
])
def test_edge_shapes(gpu_lib, shape):
    cfg = synth.VerifyConfig("edge", dtype=synth.BF16, seed=4242 + shape["N"] + shape["L"], **shape)
    x = synth.make_inputs(cfg)
    say(f"case edge {shape}")
    got, glse = gpu_dense(gpu_lib, x)
    ref, rlse = oracle_all(x)
    check_rows(got, ref, glse, rlse, cfg.dtype, str(shape))


def test_token_major_cache_and_strided_out(gpu_lib):
    cfg = synth.small_variant(C["llama3_8b_tree64_L64k"], L=500, B=2)
    x = synth.make_inputs(cfg)
    d = device_inputs(x)
    say("case token-major cache")
    kc_tm = d["k_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # [B,Hkv,L,D] view of [B,L,Hkv,D]
    vc_tm = d["v_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    out_buf = torch.zeros(cfg.B, cfg.N, cfg.Hq, cfg.D, dtype=torch.bfloat16, device="cuda")
    out = out_buf.permute(0, 2, 1, 3)
    gpu_lib.verify_attn_dense(d["q"], kc_tm, vc_tm, d["k_draft"], d["v_draft"], d["parent"], out=out)
    torch.cuda.synchronize()
    ref, _ = oracle_all(x)
    check_rows(out_to_f64(out), ref, None, None, cfg.dtype, "token-major")


def test_stages_equal_dense_and_deterministic(gpu_lib):
    cfg = synth.small_variant(C["l70b_tree128_L128k"], L=3000, B=1)
    x = synth.make_inputs(cfg)
    d = device_inputs(x)
    say("case stages + determinism")
    o1, l1 = gpu_lib.verify_attn_dense(**d)
    o2, l2 = gpu_lib.verify_attn_dense(**d)
    out = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    desc = gpu_lib.make_desc(d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], out)
    ws = torch.empty(gpu_lib.workspace_size(desc, cfg.L), dtype=torch.uint8, device="cuda")
    gpu_lib.verify_attn_partials(desc, d["q"], d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"],
                                 d["parent"], ws)
    gpu_lib.verify_attn_merge(desc, cfg.L, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), out.view(torch.int16)) and torch.equal(l1, lse)


# ---------------------------------------------------------------------------
# sparse verification and selection at small sizes


@pytest.mark.parametrize("name", ["qwen25_7b_sparse2048_L32k", "l70b_tree128_L128k"])
@pytest.mark.parametrize("L", [600, 4096])
def test_small_sparse(gpu_lib, name, L):
    cfg = synth.small_variant(C[name], L=L, B=2 if C[name].N <= 64 else 1)
    x = synth.make_inputs(cfg, scores=True)
    idx = vo.select_verify_set(x.draft_score, x.target_score, cfg.sink, cfg.window, cfg.top_m, cfg.budget)
    say(f"case sparse {cfg.name} K={idx.shape[1]}")
    got, glse = gpu_sparse(gpu_lib, x, idx)
    ref, rlse = oracle_all(x, idx=idx)
    check_rows(got, ref, glse, rlse, cfg.dtype, cfg.name)
    # and through the selector on the GPU: identical index list
    gidx = gpu_lib.select_verify_set(to_dev(x.draft_score, synth.FP32), to_dev(x.target_score, synth.FP32),
                                     sink=cfg.sink, window=cfg.window, top_m=cfg.top_m, budget=cfg.budget)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gidx.cpu().numpy(), idx)


def test_sparse_unsorted_and_all_indices(gpu_lib):
    cfg = synth.small_variant(C["qwen25_7b_sparse2048_L32k"], L=800, B=2)
    x = synth.make_inputs(cfg)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(800)[:333] for _ in range(2)]).astype(np.int32)
    say("case sparse unsorted")
    got, glse = gpu_sparse(gpu_lib, x, idx)
    ref, rlse = oracle_all(x, idx=idx)
    check_rows(got, ref, glse, rlse, cfg.dtype, "unsorted")
    say("case sparse all indices == dense")
    all_idx = np.tile(np.arange(800, dtype=np.int32), (2, 1))
    s_out, s_lse = gpu_sparse(gpu_lib, x, all_idx)
    d_out, d_lse = gpu_dense(gpu_lib, x)
    ref, rlse = oracle_all(x)
    check_rows(s_out, ref, s_lse, rlse, cfg.dtype, "all-idx")
    check_rows(d_out, ref, d_lse, rlse, cfg.dtype, "dense")


def _sel_gpu(ops, d, t, sink, window, m, budget):
    g = ops.select_verify_set(to_dev(d, synth.FP32), to_dev(t, synth.FP32), sink=sink, window=window,
                              top_m=m, budget=budget)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def test_selector_ties_specials_and_special_cases(gpu_lib):
    rng = np.random.default_rng(11)
    say("case selector ties")
    B, L = 3, 5000
    levels = np.array([np.nan, -np.inf, -0.0, 0.0, 1.0, 2.0, np.inf], dtype=np.float32)
    d = levels[rng.integers(0, len(levels), (B, L))]
    t = levels[rng.integers(0, len(levels), (B, L))]
    for (S, W, m, budget) in ((4, 256, 1024, 2048), (0, 0, 100, 100), (4, 16, 0, 500), (4, 16, 480, 500),
                              (4, 16, 10, 20), (7, 3, 9999, 4000), (4, 16, 10, L), (4, 16, 10, L + 9)):
        got = _sel_gpu(gpu_lib, d, t, S, W, m, budget)
        np.testing.assert_array_equal(got, vo.select_verify_set(d, t, S, W, m, budget), err_msg=str((S, W, m, budget)))
    say("case selector multi-segment ties, unaligned rows")
    # rows of many filter segments with a ragged last one, ties across
    # segment borders (the draft scores' few levels send the draft tier to
    # the exact way, which re-reads 32768-token segments), and a row stride
    # that leaves rows unaligned to 16 bytes
    L2, ld = 70001, 70003
    d = levels[rng.integers(2, len(levels), (2, L2))]
    t = rng.lognormal(0, 2, (2, L2)).astype(np.float32)
    t[:, 30000:40000] = 3.0
    dpad = torch.zeros(2, ld, dtype=torch.float32)
    tpad = torch.zeros(2, ld, dtype=torch.float32)
    dpad[:, :L2] = torch.from_numpy(d)
    tpad[:, :L2] = torch.from_numpy(t)
    dv, tv = dpad.cuda()[:, :L2], tpad.cuda()[:, :L2]
    # (the last three skip the draft tier, the target tier, and both)
    for (S, W, m, budget) in ((4, 256, 1024, 2048), (4, 256, 20000, 30000), (0, 100, 5, 9000),
                              (4, 256, 0, 5000), (4, 256, 50000, 3000), (4, 256, 10, 260)):
        g = gpu_lib.select_verify_set(dv, tv, sink=S, window=W, top_m=m, budget=budget)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(g.cpu().numpy(), vo.select_verify_set(d, t, S, W, m, budget),
                                      err_msg=str((S, W, m, budget)))
    say("case selector longest row (24 segments)")
    # the row length limit (192 filter segments of 4096 tokens)
    Lmax = 24 * 32768
    d = rng.lognormal(0, 2, (1, Lmax)).astype(np.float32)
    t = rng.lognormal(0, 2, (1, Lmax)).astype(np.float32)
    got = _sel_gpu(gpu_lib, d, t, 4, 256, 2048, 4096)
    np.testing.assert_array_equal(got, vo.select_verify_set(d, t, 4, 256, 2048, 4096))
    say("case selector wide batch of long rows")
    # 8 rows of 147 filter segments, a block of equal target scores
    d = rng.lognormal(0, 2, (8, 600001)).astype(np.float32)
    t = rng.lognormal(0, 2, (8, 600001)).astype(np.float32)
    t[:, 100000:100500] = 7.0
    got = _sel_gpu(gpu_lib, d, t, 4, 256, 1000, 3000)
    np.testing.assert_array_equal(got, vo.select_verify_set(d, t, 4, 256, 1000, 3000))
    say("case selector lognormal ragged")
    for L in (1, 31, 1025, 4099):
        d = rng.lognormal(0, 2, (2, L)).astype(np.float32)
        t = rng.lognormal(0, 2, (2, L)).astype(np.float32)
        for budget in (L // 3 + 2, L - 1):
            if budget < L and budget < len(vo.protected_set(L, 2, 2)):
                continue
            got = _sel_gpu(gpu_lib, d, t, 2, 2, budget // 2, budget)
            np.testing.assert_array_equal(got, vo.select_verify_set(d, t, 2, 2, budget // 2, budget))


# ---------------------------------------------------------------------------
# full workload sizes, sampled slabs


@pytest.fixture(scope="module")
def full_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            say(f"generating {name} inputs")
            cache[name] = synth.make_inputs(C[name])
        return cache[name]
    return get


def _pairs(cfg, rng):
    """(sequence, query head) pairs checked at full size: one query head of
    every (sequence, KV head) work item (a seeded choice within the group),
    plus the first and the last head of the whole batch."""
    pairs = {(0, 0), (cfg.B - 1, cfg.Hq - 1)}
    for b in range(cfg.B):
        for kvh in range(cfg.Hkv):
            pairs.add((b, kvh * cfg.G + int(rng.integers(cfg.G))))
    return sorted(pairs)


@pytest.mark.parametrize("name", ["llama3_8b_chain8_L32k", "llama3_8b_tree64_L64k", "l70b_tree128_L128k",
                                  "qwen25_7b_sparse2048_L32k"])
def test_full_size_dense_sampled(gpu_lib, full_inputs, name):
    x = full_inputs(name)
    cfg = x.cfg
    say(f"case full dense {name}")
    got, glse = gpu_dense(gpu_lib, x)
    assert np.isfinite(got).all()
    pairs = _pairs(cfg, np.random.default_rng(cfg.seed))
    assert {(b, h // cfg.G) for b, h in pairs} == {(b, k) for b in range(cfg.B) for k in range(cfg.Hkv)}
    say(f"  oracle on {len(pairs)} (sequence, head) slabs")
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, heads=pairs)
    for n, (b, h) in enumerate(pairs):
        check_rows(got[b, h], ref[n], glse[b, h], rlse[n], cfg.dtype, f"{name} b={b} h={h}")


@pytest.mark.parametrize("name", ["qwen25_7b_sparse2048_L32k", "l70b_tree128_L128k"])
def test_full_size_sparse_sampled(gpu_lib, full_inputs, name):
    x = full_inputs(name)
    cfg = x.cfg
    say(f"case full select {name}")
    idx = vo.select_verify_set(x.draft_score, x.target_score, cfg.sink, cfg.window, cfg.top_m, cfg.budget)
    gidx = _sel_gpu(gpu_lib, x.draft_score, x.target_score, cfg.sink, cfg.window, cfg.top_m, cfg.budget)
    np.testing.assert_array_equal(gidx, idx)
    say(f"case full sparse {name} K={idx.shape[1]}")
    got, glse = gpu_sparse(gpu_lib, x, idx)
    pairs = _pairs(cfg, np.random.default_rng(cfg.seed + 1))
    say(f"  oracle on {len(pairs)} (sequence, head) slabs")
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx,
                                    heads=pairs)
    for n, (b, h) in enumerate(pairs):
        check_rows(got[b, h], ref[n], glse[b, h], rlse[n], cfg.dtype, f"{name} sparse b={b} h={h}")
