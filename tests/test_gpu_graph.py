"""A verification step captured in a HIP graph.

The library's calls enqueue kernels only (no allocation, copy, fill or
host synchronisation), so a caller can capture a whole step.  The selector,
the sparse call over its output and a dense call are captured once with
preallocated outputs and workspaces; each replay then runs on new scores
and queries written into the captured input buffers, with the program's
own eager calls and synchronisations between replays, and every replay must
equal the same calls made eagerly bit for bit, and the oracle (LongSpec,
"Tree Attention Ibrida"; Dustin, "Aggregazione Ibrida dell'Attenzione").
"""

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo
from long_context_verify_tree_amd import synth
from _util import check_rows, device_inputs, out_to_f64

pytestmark = pytest.mark.gpu

SEL = dict(sink=4, window=64, top_m=256, budget=2048)


def say(*a):
    print(*a, flush=True)


def step(ops, d, ds, ts, bufs):
    """select -> sparse -> dense into the preallocated buffers bufs."""
    ops.select_verify_set(ds, ts, **SEL, out=bufs["idx"], workspace=bufs["ws_sel"])
    ops.verify_attn_sparse(**d, verify_idx=bufs["idx"], out=bufs["out_s"], lse=bufs["lse_s"],
                           workspace=bufs["ws_s"])
    ops.verify_attn_dense(**d, out=bufs["out_d"], lse=bufs["lse_d"], workspace=bufs["ws_d"])


def make_bufs(ops, d, B, L):
    q = d["q"]
    B_, Hq, N, D = q.shape
    desc = ops.make_desc(q, d["k_cache"], d["v_cache"], d["k_draft"], d["v_draft"], torch.empty_like(q))
    dev = q.device
    return dict(idx=torch.empty(B, SEL["budget"], dtype=torch.int32, device=dev),
                ws_sel=torch.empty(max(ops.select_workspace_size(B, L), 1), dtype=torch.uint8, device=dev),
                out_s=torch.empty_like(q), lse_s=torch.empty(B, Hq, N, dtype=torch.float32, device=dev),
                ws_s=torch.empty(ops.workspace_size(desc, SEL["budget"]), dtype=torch.uint8, device=dev),
                out_d=torch.empty_like(q), lse_d=torch.empty(B, Hq, N, dtype=torch.float32, device=dev),
                ws_d=torch.empty(ops.workspace_size(desc, L), dtype=torch.uint8, device=dev))


def test_captured_step_replays_match_eager(gpu_lib):
    cfg = synth.VerifyConfig("graph", B=2, Hq=8, Hkv=2, D=128, L=20000, N=16, tree="uniform", dtype=synth.BF16,
                             seed=5151)
    say("case graph: B=2 Hq=8 Hkv=2 D=128 L=20000 N=16 bf16, select -> sparse -> dense captured, 3 replays")
    x = synth.make_inputs(cfg)
    d = device_inputs(x)                   # the captured input buffers
    g = torch.Generator(device="cuda").manual_seed(29)
    ds = torch.rand(cfg.B, cfg.L, device="cuda", generator=g)
    ts = torch.rand(cfg.B, cfg.L, device="cuda", generator=g)
    cap = make_bufs(gpu_lib, d, cfg.B, cfg.L)
    eager = make_bufs(gpu_lib, d, cfg.B, cfg.L)

    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gpu_lib, d, ds, ts, cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gpu_lib, d, ds, ts, cap)
    torch.cuda.synchronize()

    q0 = d["q"].clone()
    for r in range(3):
        # new inputs in the captured buffers (eager work between replays)
        ds.copy_(torch.rand(cfg.B, cfg.L, device="cuda", generator=g))
        ts.copy_(torch.rand(cfg.B, cfg.L, device="cuda", generator=g))
        d["q"].copy_(q0 * (1.0 + 0.25 * r))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(gpu_lib, d, ds, ts, eager)
        torch.cuda.synchronize()
        for k in ("idx", "out_s", "lse_s", "out_d", "lse_d"):
            assert torch.equal(cap[k], eager[k]), f"replay {r}: {k} differs from the eager call"
        say(f"replay {r} equals the eager step")

    # the last replay against the oracle
    qn = out_to_f64(d["q"]).astype(np.float32)
    idx = cap["idx"].cpu().numpy()
    np.testing.assert_array_equal(idx, vo.select_verify_set(ds.cpu().numpy(), ts.cpu().numpy(), SEL["sink"],
                                                            SEL["window"], SEL["top_m"], SEL["budget"]))
    r_s, rl_s = vo.verify_attention(qn, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
    check_rows(out_to_f64(cap["out_s"]), r_s, cap["lse_s"].cpu().numpy().astype(np.float64), rl_s, cfg.dtype,
               "graph sparse")
    r_d, rl_d = vo.verify_attention(qn, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(out_to_f64(cap["out_d"]), r_d, cap["lse_d"].cpu().numpy().astype(np.float64), rl_d, cfg.dtype,
               "graph dense")
