"""Every call on the caller's stream.

The library enqueues all its work on the stream it is handed (the binding
passes torch's current stream).  Here the selector, the sparse call that
reads its output and a dense call run on a side stream created by torch
(which does not synchronise with the null stream), each call's inputs
produced on that same stream just before it.  Any launch that went to
another stream would race with them; the outputs must be bit-identical to
the same calls on the default stream, and match the oracle (LongSpec, "Tree
Attention Ibrida": the tree-masked attention over context and drafts;
Dustin, "Aggregazione Ibrida dell'Attenzione": the verify set).
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


def chain(ops, d, ds, ts):
    """selector -> sparse over its output -> dense, on the current stream;
    the scores are copied on this stream first, so the selector's input is
    produced by work on the same stream."""
    ds2, ts2 = ds.clone(), ts.clone()
    idx = ops.select_verify_set(ds2, ts2, **SEL)
    out_s, lse_s = ops.verify_attn_sparse(**d, verify_idx=idx)
    out_d, lse_d = ops.verify_attn_dense(**d)
    return idx, out_s, lse_s, out_d, lse_d


def test_calls_follow_the_callers_stream(gpu_lib):
    cfg = synth.VerifyConfig("streams", B=2, Hq=8, Hkv=2, D=128, L=20000, N=16, tree="uniform", dtype=synth.BF16,
                             seed=4242)
    say("case streams: B=2 Hq=8 Hkv=2 D=128 L=20000 N=16 bf16, select -> sparse -> dense on a side stream")
    x = synth.make_inputs(cfg)
    d = device_inputs(x)
    g = torch.Generator(device="cuda").manual_seed(17)
    ds = torch.rand(cfg.B, cfg.L, device="cuda", generator=g)
    ts = torch.rand(cfg.B, cfg.L, device="cuda", generator=g)
    ref = chain(gpu_lib, d, ds, ts)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = chain(gpu_lib, d, ds, ts)
    side.synchronize()
    for name, a, b in zip(("verify_idx", "sparse out", "sparse lse", "dense out", "dense lse"), ref, got):
        assert torch.equal(a, b), f"{name} differs between the default and the side stream"

    idx = ref[0].cpu().numpy()
    np.testing.assert_array_equal(idx, vo.select_verify_set(ds.cpu().numpy(), ts.cpu().numpy(), SEL["sink"],
                                                            SEL["window"], SEL["top_m"], SEL["budget"]))
    r_s, rl_s = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx)
    check_rows(out_to_f64(got[1]), r_s, got[2].cpu().numpy().astype(np.float64), rl_s, cfg.dtype, "side stream sparse")
    r_d, rl_d = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(out_to_f64(got[3]), r_d, got[4].cpu().numpy().astype(np.float64), rl_d, cfg.dtype, "side stream dense")


def test_two_streams_with_own_workspaces(gpu_lib):
    # calls that overlap in time on two streams, each with its own outputs
    # and workspace, give what the same calls give one after another
    say("case two streams: two problems, select -> sparse -> dense on each of two side streams at once")
    probs = []
    for seed in (606, 707):
        cfg = synth.VerifyConfig("streams2", B=2, Hq=8, Hkv=2, D=128, L=20000, N=16, tree="uniform",
                                 dtype=synth.BF16, seed=seed)
        x = synth.make_inputs(cfg)
        g = torch.Generator(device="cuda").manual_seed(seed)
        probs.append((device_inputs(x), torch.rand(cfg.B, cfg.L, device="cuda", generator=g),
                      torch.rand(cfg.B, cfg.L, device="cuda", generator=g)))
    ref = [chain(gpu_lib, *p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                got[i] = chain(gpu_lib, *probs[i])
        for s in streams:
            s.synchronize()
        for i in range(2):
            for name, a, b in zip(("verify_idx", "sparse out", "sparse lse", "dense out", "dense lse"), ref[i], got[i]):
                assert torch.equal(a, b), f"repeat {rep}, problem {i}: {name} differs from the serial call"
