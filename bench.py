"""Benchmark of speculative-verification attention on one MI355X.

One step = one verification pass of one target-model layer over the whole
batch, through the C ABI: the partial kernel (context splits + tree part) and
the log-sum-exp merge; for a sparse workload the step also runs the verify-set
selector.  Inputs are seeded synthetic tensors of the workload's shape
(long_context_verify_tree_amd.synth), resident in HBM before timing starts;
at least four copies are rotated, and enough that a copy is read again only
after more than twice the 256 MB MALL of other inputs, so no step reuses
cached data.

Prints one JSON line.  `value` is the algorithmic HBM throughput of the whole
step in GB/s (bytes the method must move / step time); the same line carries
draft tokens verified per second per layer, the roofline fraction of the
dominant kernel (timed with HIP events on the stream it runs on) and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0 # dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3
DEFAULT_CONFIG = "l70b_tree128_L128k"


def algorithmic(cfg, n_ctx: int, sparse: bool):
    """Bytes and flops the method must move / compute for one step."""
    e = 4 if cfg.dtype == "fp32" else 2
    B, Hq, Hkv, D, N = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.N
    kv = 2 * B * Hkv * n_ctx * D * e
    q = B * Hq * N * D * e
    draft = 2 * B * Hkv * N * D * e
    out = B * Hq * N * D * e + B * Hq * N * 4
    idx = B * n_ctx * 4 if sparse else 0
    parent = B * N * 4
    flops = 4 * B * Hq * N * n_ctx * D
    return dict(kv=kv, partial_bytes=kv + q + draft + parent + idx, step_bytes=kv + q + draft + out + idx + parent,
                flops=flops)


CSRC = os.path.join(ROOT, "long_context_verify_tree_amd", "csrc")
KERNEL_SOURCES = {"partial_kernel": "va_attn.hip", "rows_kernel": "va_attn.hip", "select_filter_kernel": "va_select.hip",
                  "select_resolve_kernel": "va_select.hip", "score_partial_kernel": "va_score.hip"}


def committed_summary(kernel: str, workload: str, suffix: str = ""):
    """Fields of the committed rocprofv3 summary profiles/<kernel>_<workload><suffix>.md
    as (fields, path), or (None, note) if there is none or the kernel source
    changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}{suffix}.md")
    if not os.path.exists(path):
        return None, None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    # the kernel's source file, then the device header every kernel includes
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "va_device.h"):
        h.update(open(os.path.join(CSRC, name), "rb").read())
    if fields.get("kernel source sha256") != h.hexdigest():
        return None, os.path.relpath(path, ROOT) + " (stale: kernel changed since the counters were taken)"
    return fields, os.path.relpath(path, ROOT)


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None if there is none or the kernel source changed since."""
    fields, src = committed_summary(kernel, workload)
    if fields is None or "traffic bytes per launch" not in fields:
        return None, src
    return int(float(fields["traffic bytes per launch"])), src


def committed_mfma_util(kernel: str, workload: str):
    """MFMA-busy percentage (rocprofv3's MfmaUtil) of `kernel` from the
    committed pipe-counter summary, or None (missing or stale)."""
    fields, src = committed_summary(kernel, workload, "_pipes")
    if fields is None or "mfma util percent" not in fields:
        return None, src
    return float(fields["mfma util percent"]), src


def attention_kernel(cfg) -> str:
    """Which partial kernel the library picks: the shared-tile kernel for bf16
    with more than 64 query rows per KV head, the per-wavefront kernel else."""
    return "rows_kernel" if cfg.dtype == "bf16" and cfg.G * cfg.N > 64 else "partial_kernel"


def select_kernel_name(B: int, L: int, budget: int) -> str:
    """The selector's kernels: a filter over many workgroups per row, then one
    resolving workgroup per row; with budget >= L only the second runs (every
    index is taken)."""
    return "select_filter_kernel+select_resolve_kernel" if budget < L else "select_resolve_kernel"


def verify_mode(cfg, verify: str) -> bool:
    """True for a sparse step.  `auto` takes the workload's own mode (sparse
    only when it has no dense run); `dense` / `sparse` pick one explicitly."""
    if verify == "auto":
        return cfg.sparse and not cfg.dense
    if verify == "sparse" and not cfg.sparse:
        raise SystemExit(f"{cfg.name} has no verify-set parameters")
    return verify == "sparse"


def workload_name(cfg, sparse: bool) -> str:
    """The workload's name, with the verify mode appended when it is not the
    workload's own (the 70B-shape sparse run, the Qwen-shape dense run)."""
    if sparse == (cfg.sparse and not cfg.dense):
        return cfg.name
    return f"{cfg.name}_sparse{cfg.budget}" if sparse else f"{cfg.name}_dense"


def measured_read_peak(torch, dev, gib: float = 2.0, reps: int = 10, min_seconds: float = 0.4):
    """Achievable HBM read bandwidth (GB/s) from the read-only probe library.
    Also keeps the GPU busy for at least `min_seconds` first, so the timed
    steps that follow run at a settled clock."""
    import ctypes
    path = os.path.join(ROOT, "long_context_verify_tree_amd", "libva_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.va_probe_hbm_read.restype = ctypes.c_int
    lib.va_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    n = int(gib * (1 << 30))
    buf = torch.ones(n // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    t_end = time.perf_counter() + min_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            lib.va_probe_hbm_read(buf.data_ptr(), n, sink.data_ptr(), 256 * 16, stream)
        torch.cuda.synchronize()
    best = 0.0
    for grid in (256 * 8, 256 * 16, 256 * 32):
        def run():
            rc = lib.va_probe_hbm_read(buf.data_ptr(), n, sink.data_ptr(), grid, stream)
            if rc != 0:
                raise RuntimeError(f"va_probe_hbm_read failed: {rc}")
        run()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            run()
        b.record()
        b.synchronize()
        best = max(best, reps * n / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return round(best, 1)


def measured_gather_peak(torch, sets, idx_bufs, cfg, n_ctx: int, reps: int = 8):
    """Achievable rate (GB/s) of the sparse step's gathered K/V reads: the
    probe library reads the same rows (each input copy with the index list
    selected for it, copies rotated as in the timed steps) with no compute."""
    import ctypes
    path = os.path.join(ROOT, "long_context_verify_tree_amd", "libva_probe.so")
    if not os.path.exists(path) or n_ctx <= 0:
        return None
    lib = ctypes.CDLL(path)
    fn = lib.va_probe_gather_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p,
                                                                                             ctypes.c_int,
                                                                                             ctypes.c_void_p]
    e = 4 if cfg.dtype == "fp32" else 2
    row_bytes = cfg.D * e
    for st in sets:   # the probe takes [B, Hkv, L, D] rows back to back
        assert st["k_cache"].is_contiguous() and st["v_cache"].is_contiguous()
    for ib in idx_bufs:
        assert ib.is_contiguous() and ib.shape == (cfg.B, n_ctx)
    sink = torch.zeros(1, dtype=torch.int32, device=sets[0]["k_cache"].device)
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 2 * cfg.B * cfg.Hkv * n_ctx * row_bytes
    best = 0.0
    for grid in (256 * 8, 256 * 16, 256 * 32):
        def run(i):
            st = sets[i % len(sets)]
            rc = fn(st["k_cache"].data_ptr(), st["v_cache"].data_ptr(), idx_bufs[i % len(sets)].data_ptr(), cfg.B,
                    cfg.Hkv, n_ctx, cfg.L, row_bytes, sink.data_ptr(), grid, stream)
            if rc != 0:
                raise RuntimeError(f"va_probe_gather_read failed: {rc}")
        run(0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            run(i + 1)
        b.record()
        b.synchronize()
        best = max(best, reps * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    return round(best, 1)


def cpu_baseline(cfg, x, budget_s: float, sparse: bool):
    """The oracle, untouched, on as many (sequence, KV-head group) slabs of the
    benchmarked inputs as fit the time budget."""
    from threadpoolctl import threadpool_info
    from oracle import verify_oracle as vo

    t0 = time.perf_counter()
    idx = None
    if sparse:
        idx = vo.select_verify_set(x.draft_score, x.target_score, cfg.sink, cfg.window, cfg.top_m, cfg.budget)
    groups = [(b, kvh) for b in range(cfg.B) for kvh in range(cfg.Hkv)]
    done = 0
    while done < len(groups) and time.perf_counter() - t0 < budget_s:
        b, kvh = groups[done]
        vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent, ctx_index=idx,
                            heads=[(b, kvh * cfg.G + g) for g in range(cfg.G)])
        done += 1
    dt = time.perf_counter() - t0
    n_ctx = min(cfg.budget, cfg.L) if sparse else cfg.L
    frac = done / len(groups)
    sample_bytes = algorithmic(cfg, n_ctx, sparse)["step_bytes"] * frac
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {
        "value": round(sample_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s_per_layer": round(cfg.B * cfg.N * frac / dt, 3),
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done}/{len(groups)} (sequence, KV head) slabs of the benchmarked {workload_name(cfg, sparse)} inputs"
                  f"{' incl. selection' if sparse else ''}, fp64 numpy, {dt:.1f} s",
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_commit(torch, ops, cfg, x, base, dev, reps: int = 20):
    """Accept-and-commit of the deepest draft node of every sequence (its
    whole root path) into the last rows of the benchmarked cache; mean of
    `reps` launches timed with HIP events on the launching stream.  Runs
    after the timed steps (it overwrites cache rows)."""
    depth = np.zeros((cfg.B, cfg.N), dtype=np.int64)
    for b in range(cfg.B):
        for i in range(cfg.N):
            p = int(x.parent[b, i])
            depth[b, i] = 1 if p < 0 else depth[b, p] + 1
    leaf = depth.argmax(axis=1)
    plen = depth.max(axis=1)
    accepted = torch.from_numpy(leaf.astype(np.int32)).to(dev)
    cache_len = torch.from_numpy((cfg.L - plen).astype(np.int32)).to(dev)
    new_len = torch.empty(cfg.B, dtype=torch.int32, device=dev)
    args = (base["k_cache"], base["v_cache"], base["k_draft"], base["v_draft"], base["parent"], accepted, cache_len,
            new_len)
    desc = ops.make_commit_desc(*args[:4])
    ops.accept_commit(*args)
    torch.cuda.synchronize()
    a, bev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ops.accept_commit(*args, desc=desc)
    bev.record()
    bev.synchronize()
    us = a.elapsed_time(bev) * 1e3 / reps
    e = 4 if cfg.dtype == "fp32" else 2
    nbytes = int(2 * 2 * cfg.Hkv * cfg.D * e * int(plen.sum()))   # K and V rows, read once and written once
    return {"us": round(us, 2), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 2),
            "rows_per_sequence": int(plen.max()), "kernel": "commit_kernel"}


SCORE_HEADS = 2   # scoring heads of the importance map (a few selected heads)


def measure_scores(torch, ops, cfg, sets, dev, step_ms, reps: int = 20):
    """Importance map of SCORE_HEADS scoring heads with (up to 32 of) the
    draft rows each, over the benchmarked cache's first KV heads; mean of
    `reps` calls timed with HIP events on the launching stream.  The calls
    rotate over the input copies as the verification steps do, so the
    scoring heads' K rows come from HBM, not from the 256 MB MALL."""
    if cfg.dtype != "bf16" or cfg.L == 0:
        return None
    hs = min(SCORE_HEADS, cfg.Hkv)
    rows = min(cfg.N, 32)                      # scoring rows per head (the kernel takes up to 32)
    qs = [st["q"][:, :hs, :rows] for st in sets]
    ks = [st["k_cache"][:, :hs] for st in sets]
    desc = ops.make_score_desc(qs[0], ks[0])
    ws = torch.empty(ops.scores_workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty(cfg.B, cfg.L, dtype=torch.float32, device=dev)
    ops.importance_scores(qs[0], ks[0], out=out, workspace=ws, desc=desc)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        j = (i + 1) % len(sets)
        ops.importance_scores(qs[j], ks[j], out=out, workspace=ws, desc=desc)
    b.record()
    b.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = cfg.B * hs * (cfg.L + rows) * cfg.D * 2 + cfg.B * cfg.L * 4   # K and q read, map written
    return {"us": round(us, 2), "bytes": nbytes, "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "scoring_heads": hs, "rows_per_head": rows, "input_copies_rotated": len(sets),
            "vs_one_verification_step": round(us * 1e-3 / step_ms, 4),
            "kernels": ["score_partial_kernel", "score_finish_kernel"]}


TREE_POSITIONS, TREE_CANDIDATES = 16, 8   # block positions and candidates per position of the drafter


def measure_tree(torch, ops, cfg, dev, reps: int = 20):
    """Best-first draft tree of the workload's N nodes per sequence from
    seeded synthetic candidates (Dirichlet(0.3) marginals over
    TREE_CANDIDATES tokens at each of TREE_POSITIONS positions)."""
    rng = np.random.default_rng(cfg.seed + 9)
    K, T = TREE_POSITIONS, TREE_CANDIDATES
    prob = torch.from_numpy(rng.dirichlet(np.full(T, 0.3), size=(cfg.B, K)).astype(np.float32)).to(dev)
    tok = torch.from_numpy(rng.integers(0, 1 << 17, (cfg.B, K, T)).astype(np.int32)).to(dev)
    res = ops.build_draft_tree(prob, tok, cfg.N)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ops.build_draft_tree(prob, tok, cfg.N)
    b.record()
    b.synchronize()
    return {"us": round(a.elapsed_time(b) * 1e3 / reps, 2), "nodes": cfg.N, "positions": K, "candidates": T,
            "mean_a_hat": round(float(res[3].mean().item()), 4), "kernel": "tree_kernel"}


SWEEP_N = (1, 2, 4, 8, 12, 16, 17, 24, 32, 48, 64, 65, 96, 128, 129, 160, 192, 224, 256)


def sweep_n(args):
    """T_verify(N) on the workload's context (K/V cache, batch, heads) for
    best-first trees of N nodes built from synthetic drafter candidates;
    least-squares calibration of the library's plan-following time model
    (bandwidth, the two kernels' compute rates, overhead); the knee where the
    model turns compute-bound; the controller's tree size on the trees'
    surrogate curve."""
    import torch
    from scipy.optimize import least_squares
    from long_context_verify_tree_amd import ops, synth

    ops.load()
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, Hq, Hkv, D, L = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.L
    kc = torch.randn(B, Hkv, L, D, device=dev, generator=g).to(dt)
    vc = torch.randn(B, Hkv, L, D, device=dev, generator=g).to(dt)
    # best-first trees of up to 256 nodes from seeded drafter candidates
    rng = np.random.default_rng(cfg.seed + 9)
    K, T = TREE_POSITIONS, TREE_CANDIDATES
    prob = torch.from_numpy(rng.dirichlet(np.full(T, 0.3), size=(B, K)).astype(np.float32)).to(dev)
    tok = torch.from_numpy(rng.integers(0, 1 << 17, (B, K, T)).astype(np.int32)).to(dev)
    read_peak = measured_read_peak(torch, dev)
    times = []
    for N in SWEEP_N:
        parent, _, rho, _ = ops.build_draft_tree(prob, tok, N)
        q = torch.randn(B, Hq, N, D, device=dev, generator=g).to(dt)
        kd = torch.randn(B, Hkv, N, D, device=dev, generator=g).to(dt)
        vd = torch.randn(B, Hkv, N, D, device=dev, generator=g).to(dt)
        out = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device=dev)
        desc = ops.make_desc(q, kc, vc, kd, vd, out)
        ws = torch.empty(ops.workspace_size(desc, L), dtype=torch.uint8, device=dev)

        def step():
            ops.verify_attn_partials(desc, q, kc, vc, kd, vd, parent, ws)
            ops.verify_attn_merge(desc, L, out, lse, ws)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) / args.steps)
        print(f"[sweep] N={N}: {times[-1] * 1e3:.4f} ms", file=sys.stderr, flush=True)
    rho_all = ops.build_draft_tree(prob, tok, SWEEP_N[-1])[2].cpu().numpy().astype(np.float64)
    a_curve = np.cumsum(rho_all.mean(axis=0))          # surrogate of the best-first tree of n nodes
    desc1 = ops.make_desc(torch.empty(B, Hq, 1, D, dtype=dt, device=dev), kc, vc,
                          torch.empty(B, Hkv, 1, D, dtype=dt, device=dev), torch.empty(B, Hkv, 1, D, dtype=dt, device=dev),
                          torch.empty(B, Hq, 1, D, dtype=dt, device=dev))

    def model(p, ns):
        bw, cs, ct, c0 = np.exp(p)
        return np.array([ops.verify_time_model(desc1, L, bw, cs, ct, c0, int(n)) for n in ns])
    ns = np.array(SWEEP_N)
    ts = np.array(times)
    # least squares on log times from several starting points: the max() of
    # the model leaves flat directions (a compute rate that never binds), where
    # one start can stop far from the best fit; keep the smallest worst residual
    fit, worst = None, None
    for ct0, cs0 in ((1e14, 5e14), (1e14, 1e15), (1e14, 2e15), (4e14, 1e15), (1e15, 1e15), (1e15, 2e15)):
        f = least_squares(lambda p: np.log(model(p, ns)) - np.log(ts), x0=np.log([5e12, cs0, ct0, 5e-6]),
                          bounds=(np.log([1e11, 1e12, 1e12, 1e-8]), np.log([2e13, 5e15, 5e15, 1e-2])))
        w = float(np.max(np.abs(model(f.x, ns) / ts - 1)))
        if worst is None or w < worst:
            fit, worst = f, w
    bw, cs, ct, c0 = (float(v) for v in np.exp(fit.x))
    n_all = np.arange(1, SWEEP_N[-1] + 1)
    t_model = model(fit.x, n_all)
    # knee: the first N whose padded MFMA work outlasts the K/V stream in the fitted model
    e = 2 if cfg.dtype == "bf16" else 4
    kv_t = 2.0 * B * Hkv * L * D * e / bw
    knee = 0
    for n in n_all:
        t_no_compute = ops.verify_time_model(desc1, L, bw, 1e30, 1e30, c0, int(n))
        if t_model[n - 1] > t_no_compute * (1 + 1e-9):
            knee = int(n)
            break
    t_ar = float(t_model[0])                           # one autoregressive step's verification
    n_best = ops.choose_tree_size(a_curve, t_model, t_draft=t_ar, l_ar=t_ar)
    S = a_curve * t_ar / (t_ar + t_model)
    resid = model(fit.x, ns) / ts - 1
    line = {
        "metric": "T_verify(N) sweep + tree-size controller",
        "workload": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "n_ctx_keys": L,
        "dtype": cfg.dtype, "steps": args.steps, "warmup": args.warmup,
        "N": list(SWEEP_N), "t_verify_ms": [round(t * 1e3, 4) for t in times],
        "t_model_ms": [round(float(t) * 1e3, 4) for t in model(fit.x, ns)],
        "fit": {"model": "max(KV / bw, padded flops / compute_kernel) + partial rows / bw + overhead (kernel plan)",
                "bandwidth_gbs": round(bw / 1e9, 1), "compute_shared_tflops": round(cs / 1e12, 1),
                "compute_tiles_tflops": round(ct / 1e12, 1), "overhead_us": round(c0 * 1e6, 2),
                "max_rel_residual": round(float(np.max(np.abs(resid))), 4),
                "kv_stream_ms": round(kv_t * 1e3, 4)},
        "knee_N": knee, "measured_read_peak_gbs": read_peak,
        "controller": {"t_draft": "= T_verify(1)", "l_ar": "= T_verify(1)", "n_best": n_best,
                       "a_hat_at_n_best": round(float(a_curve[n_best - 1]), 4),
                       "speedup_estimate_at_n_best": round(float(S[n_best - 1]), 4),
                       "tree": f"best-first from Dirichlet(0.3) marginals, {TREE_POSITIONS} positions x "
                               f"{TREE_CANDIDATES} candidates"},
    }
    print(json.dumps(line), flush=True)


CROSSOVER_L = (2048, 4096, 8192, 16384, 32768)


def score_crossover(args):
    """Cost of importance estimation against full-cache verification as the
    context grows (Dustin, "Definizione del Problema": estimators that
    materialise scores over every head cost more than full attention beyond
    about 4k tokens; "Metodologia" section 2: scoring a few heads costs a
    small fraction).  On the workload's head shape, for each L: dense
    verification (partials + merge), the scoring pass of SCORE_HEADS heads x
    (up to 32) draft rows, and a naive estimator that scores every query row
    of every head (the importance map of all Hq * N rows); HIP events on the
    launching stream, rotated input copies."""
    import torch
    from long_context_verify_tree_amd import ops, synth

    ops.load()
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 3)
    dt = torch.bfloat16
    B, Hq, Hkv, D, N = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.N
    G = Hq // Hkv
    rows_all = G * N
    reps, copies = 10, 4
    res = []
    for L in CROSSOVER_L:
        sets = []
        for _ in range(copies):
            sets.append(dict(q=torch.randn(B, Hq, N, D, device=dev, generator=g).to(dt),
                             kc=torch.randn(B, Hkv, L, D, device=dev, generator=g).to(dt),
                             vc=torch.randn(B, Hkv, L, D, device=dev, generator=g).to(dt),
                             kd=torch.randn(B, Hkv, N, D, device=dev, generator=g).to(dt),
                             vd=torch.randn(B, Hkv, N, D, device=dev, generator=g).to(dt)))
        parent = torch.from_numpy(np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))).to(dev)
        out = torch.empty_like(sets[0]["q"])
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device=dev)
        desc = ops.make_desc(sets[0]["q"], sets[0]["kc"], sets[0]["vc"], sets[0]["kd"], sets[0]["vd"], out)
        ws = torch.empty(ops.workspace_size(desc, L), dtype=torch.uint8, device=dev)
        hs = min(SCORE_HEADS, Hkv)
        srow = min(N, 32)
        sdesc = ops.make_score_desc(sets[0]["q"][:, :hs, :srow], sets[0]["kc"][:, :hs])
        sws = torch.empty(ops.scores_workspace_size(sdesc), dtype=torch.uint8, device=dev)
        smap = torch.empty(B, L, dtype=torch.float32, device=dev)
        # the naive estimator: every query row of every head, 32 rows a call
        ndescs = []
        for r0 in range(0, rows_all, 32):
            qq = sets[0]["q"].reshape(B, Hkv, rows_all, D)[:, 0:1, r0:r0 + 32]
            ndescs.append((r0, ops.make_score_desc(qq, sets[0]["kc"][:, 0:1])))
        nws = torch.empty(max(ops.scores_workspace_size(d) for _, d in ndescs), dtype=torch.uint8, device=dev)

        def attn(st):
            ops.verify_attn_partials(desc, st["q"], st["kc"], st["vc"], st["kd"], st["vd"], parent, ws)
            ops.verify_attn_merge(desc, L, out, lse, ws)

        def srh(st):
            ops.importance_scores(st["q"][:, :hs, :srow], st["kc"][:, :hs], out=smap, workspace=sws, desc=sdesc)

        def naive(st):
            qr = st["q"].reshape(B, Hkv, rows_all, D)
            for kvh in range(Hkv):
                for r0, d in ndescs:
                    ops.importance_scores(qr[:, kvh:kvh + 1, r0:r0 + 32], st["kc"][:, kvh:kvh + 1], out=smap,
                                          workspace=nws, desc=d)

        def timed(fn):
            for i in range(3):
                fn(sets[i % copies])
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                fn(sets[(i + 1) % copies])
            b.record()
            b.synchronize()
            return a.elapsed_time(b) * 1e3 / reps
        t_attn, t_srh, t_naive = timed(attn), timed(srh), timed(naive)
        res.append({"L": L, "verify_us": round(t_attn, 2), "scoring_heads_us": round(t_srh, 2),
                    "all_heads_us": round(t_naive, 2), "scoring_heads_vs_verify": round(t_srh / t_attn, 4),
                    "all_heads_vs_verify": round(t_naive / t_attn, 4)})
        print(f"[crossover] L={L}: {res[-1]}", file=sys.stderr, flush=True)
        del sets, ws
    cross = next((r["L"] for r in res if r["all_heads_us"] > r["verify_us"]), None)
    print(json.dumps({"metric": "importance estimation cost vs full-cache verification",
                      "workload_head_shape": cfg.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                      "draft_nodes": N, "scoring_heads": min(SCORE_HEADS, Hkv), "points": res,
                      "all_heads_first_L_above_verify": cross}), flush=True)


def run_steps(torch, ops, cfg, sparse: bool, sets, dev, steps: int, warmup: int):
    """Times `steps` whole verification steps (selector when sparse, partials,
    merge) of one mode over the rotated input copies, after `warmup` untimed
    ones; then the same steps again with HIP events on the launching stream
    around each stage.  Returns the timings and the buffers of the last step."""
    n_ctx = min(cfg.budget, cfg.L) if sparse else cfg.L
    base = sets[0]
    out = torch.empty_like(base["q"])
    lse = torch.empty(cfg.B, cfg.Hq, cfg.N, dtype=torch.float32, device=dev)
    desc = ops.make_desc(base["q"], base["k_cache"], base["v_cache"], base["k_draft"], base["v_draft"], out)
    ws = torch.empty(ops.workspace_size(desc, n_ctx), dtype=torch.uint8, device=dev)
    idx_bufs = [torch.empty(cfg.B, n_ctx, dtype=torch.int32, device=dev) for _ in sets] if sparse else None
    sel_ws = (torch.empty(max(ops.select_workspace_size(cfg.B, cfg.L), 1), dtype=torch.uint8, device=dev)
              if sparse else None)

    def step(i, ev=None):
        s = sets[i % len(sets)]
        if ev is not None:
            ev[0].record()
        idx = None
        if sparse:
            idx = ops.select_verify_set(s["draft_score"], s["target_score"], sink=cfg.sink, window=cfg.window,
                                        top_m=cfg.top_m, budget=cfg.budget, out=idx_bufs[i % len(sets)],
                                        workspace=sel_ws)
        if ev is not None:
            ev[1].record()
        ops.verify_attn_partials(desc, s["q"], s["k_cache"], s["v_cache"], s["k_draft"], s["v_draft"],
                                 s["parent"], ws, verify_idx=idx)
        if ev is not None:
            ev[2].record()
        ops.verify_attn_merge(desc, n_ctx, out, lse, ws)
        if ev is not None:
            ev[3].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(warmup + steps + i, evs[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    return dict(n_ctx=n_ctx, ms_per_step=wall * 1e3 / steps, wall_ev=wall_ev,
                sel_ms=[e[0].elapsed_time(e[1]) for e in evs], part_ms=[e[1].elapsed_time(e[2]) for e in evs],
                merge_ms=[e[2].elapsed_time(e[3]) for e in evs], idx_bufs=idx_bufs, sel_ws=sel_ws)


def _pct(xs, q):
    return round(float(np.percentile(xs, q)), 4)


def roofline_of(cfg, sparse: bool, r, read_peak, wname):
    """The roofline object of the dominant kernel of one mode's steps: the
    partial (or rows) kernel, or the selector when it is slower."""
    n_ctx = r["n_ctx"]
    a = algorithmic(cfg, n_ctx, sparse)
    part_avg = statistics.mean(r["part_ms"])
    sel_avg = statistics.mean(r["sel_ms"]) if sparse else 0.0
    if sparse and sel_avg > part_avg:
        # the selector dominates: an HBM scan of both score rows plus the index write
        kernel = select_kernel_name(cfg.B, cfg.L, cfg.budget)
        sel_bytes = 2 * cfg.B * cfg.L * 4 + cfg.B * n_ctx * 4
        ach = sel_bytes / (sel_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
        roof["kernel_avg_us"] = round(sel_avg * 1e3, 2)
        roof["algorithmic_bytes_per_launch"] = sel_bytes
    else:
        kernel = attention_kernel(cfg)
        achieved = a["partial_bytes"] / (part_avg * 1e-3) / 1e9
        flops_rate = a["flops"] / (part_avg * 1e-3) / 1e12
        mfma_bound = a["flops"] / a["partial_bytes"] > (MFMA_BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9)
        if mfma_bound:
            roof = {"bound": "mfma", "achieved": round(flops_rate, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(flops_rate / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
        else:
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
        roof["kernel_avg_us"] = round(part_avg * 1e3, 2)
        roof["kernel_p10_p90_us"] = [round(_pct(r["part_ms"], 10) * 1e3, 2), round(_pct(r["part_ms"], 90) * 1e3, 2)]
        roof["algorithmic_bytes_per_launch"] = a["partial_bytes"]
        roof["algorithmic_flops_per_launch"] = a["flops"]
        roof["hbm_gbs"] = round(achieved, 1)
        if read_peak:
            roof["frac_of_measured_read_peak"] = round(achieved / read_peak, 4)
    roof["kernel"] = kernel
    roof["measured_read_peak_gbs"] = read_peak
    roof["traffic"], roof["traffic_source"] = committed_traffic(kernel, wname)
    # cross-check of the MFMA share: the MFMA pipe's busy fraction from rocprofv3 counters, where taken
    mfma_pct, mfma_src = committed_mfma_util(kernel, wname)
    if mfma_src is not None:
        roof["mfma_busy_counter_pct"], roof["mfma_counter_source"] = mfma_pct, mfma_src
    return roof


def sparse_extras(torch, ops, cfg, sets, r, es):
    """Selector figures and the gathered-read ceiling of a sparse mode."""
    n_ctx = r["n_ctx"]
    idx_bufs = r["idx_bufs"]
    for i, st in enumerate(sets):   # every copy's index list, as its steps select it
        ops.select_verify_set(st["draft_score"], st["target_score"], sink=cfg.sink, window=cfg.window,
                              top_m=cfg.top_m, budget=cfg.budget, out=idx_bufs[i], workspace=r["sel_ws"])
    torch.cuda.synchronize()
    gpeak = measured_gather_peak(torch, sets, idx_bufs, cfg, n_ctx)
    a = algorithmic(cfg, n_ctx, True)
    part_avg = statistics.mean(r["part_ms"])
    sel_avg = statistics.mean(r["sel_ms"])
    att_gbs = a["partial_bytes"] / (part_avg * 1e-3) / 1e9
    gather = {"gbs": gpeak, "bytes_per_call": 2 * cfg.B * cfg.Hkv * n_ctx * cfg.D * es,
              "attention_kernel": attention_kernel(cfg), "attention_kernel_gbs": round(att_gbs, 1),
              "attention_frac_of_gather_probe": round(att_gbs / gpeak, 4) if gpeak else None}
    sel_bytes = 2 * cfg.B * cfg.L * 4 + cfg.B * n_ctx * 4
    selector = {"kernel": select_kernel_name(cfg.B, cfg.L, cfg.budget), "us": round(sel_avg * 1e3, 2),
                "p10_p90_us": [round(_pct(r["sel_ms"], 10) * 1e3, 2), round(_pct(r["sel_ms"], 90) * 1e3, 2)],
                "bytes": sel_bytes, "gbs": round(sel_bytes / (sel_avg * 1e-3) / 1e9, 1),
                "share_of_step": round(sel_avg / r["ms_per_step"], 4)}
    # Attention Recovery Rate of the first copy's verify set for its own
    # verification rows (diagnostic: the synthetic scores are unrelated to
    # q.k, so it sits near the set's share of the cache)
    arr = ops.attention_recovery(sets[0]["q"], sets[0]["k_cache"], idx_bufs[0])
    torch.cuda.synchronize()
    selector["attention_recovery_mean"] = round(float(arr.mean().item()), 4)
    selector["set_share_of_cache"] = round(n_ctx / cfg.L, 4)
    return gather, selector


def stage_summary(r, sparse):
    return {"select": round(statistics.median(r["sel_ms"]), 4) if sparse else 0.0,
            "partials": round(statistics.median(r["part_ms"]), 4),
            "merge": round(statistics.median(r["merge_ms"]), 4),
            "partials_p10_p90": [_pct(r["part_ms"], 10), _pct(r["part_ms"], 90)],
            "instrumented_step": round(r["wall_ev"] * 1e3 / len(r["part_ms"]), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--verify", choices=("auto", "dense", "sparse"), default="auto",
                    help="dense or sparse (verify-set) context; auto: the workload's own mode")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated over steps (0: auto)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-mode", action="store_true",
                    help="skip the second verify mode of a workload that has both (dense and sparse)")
    ap.add_argument("--sweep-n", action="store_true",
                    help="instead of the step benchmark: time verification for N = 1..256 draft nodes on the "
                         "workload's cache, calibrate the roofline time model and run the tree-size controller")
    ap.add_argument("--score-crossover", action="store_true",
                    help="instead of the step benchmark: importance estimation (a few scoring heads, and every "
                         "head) against dense verification for L = 2k..32k on the workload's head shape")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the read-only HBM probe (counter-collection runs)")
    ap.add_argument("--copy-calib-gib", type=float, default=0.0,
                    help="after timing, run a plain device copy of this many GiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the kernels use no collectives",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep_n:
        sweep_n(args)
        return
    if args.score_crossover:
        score_crossover(args)
        return

    import torch
    from long_context_verify_tree_amd import ops, synth

    ops.load()
    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sparse = verify_mode(cfg, args.verify)
    wname = workload_name(cfg, sparse)
    # the workload's other verify mode (the 70B-shape sparse run beside its dense headline)
    other = None
    if args.verify == "auto" and cfg.sparse and cfg.dense and not args.no_other_mode:
        other = not sparse
    need_scores = sparse or other is True
    print(f"[bench] generating {wname}", file=sys.stderr, flush=True)
    x = synth.make_inputs(cfg, scores=need_scores)

    def dv(a, dt):
        if dt == synth.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = dict(q=dv(x.q, cfg.dtype), k_cache=dv(x.k_cache, cfg.dtype), v_cache=dv(x.v_cache, cfg.dtype),
                k_draft=dv(x.k_draft, cfg.dtype), v_draft=dv(x.v_draft, cfg.dtype),
                parent=torch.from_numpy(x.parent).to(dev))
    if need_scores:
        base["draft_score"] = dv(x.draft_score, synth.FP32)
        base["target_score"] = dv(x.target_score, synth.FP32)
    # Bytes one step reads from its input copy (gathered rows and scores when
    # sparse).  At least four copies rotate, and enough that a copy is read
    # again only after more than twice the 256 MB MALL of other inputs.
    es = 4 if cfg.dtype == "fp32" else 2

    def copies_for(sp):
        n_keys = min(cfg.budget, cfg.L) if sp else cfg.L
        step_read = 2 * cfg.B * cfg.Hkv * n_keys * cfg.D * es + (2 * cfg.B * cfg.L * 4 if sp else 0)
        return int(min(16, max(4, 1 + np.ceil(512e6 / max(step_read, 1)))))
    copies = args.copies or max(copies_for(sparse), copies_for(other) if other is not None else 0)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]

    # achievable read bandwidth; this also brings the clock up before warm-up
    read_peak = None if args.no_read_probe else measured_read_peak(torch, dev)
    r = run_steps(torch, ops, cfg, sparse, sets, dev, args.steps, args.warmup)
    n_ctx = r["n_ctx"]
    ms_per_step = r["ms_per_step"]
    a = algorithmic(cfg, n_ctx, sparse)
    value = a["step_bytes"] / (ms_per_step * 1e-3) / 1e9
    roof = roofline_of(cfg, sparse, r, read_peak, wname)

    line = {
        "metric": "verify-attention HBM GB/s (% of peak) + draft tokens verified/sec per layer",
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "draft_tokens_verified_per_s_per_layer": round(cfg.B * cfg.N / (ms_per_step * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "stage_ms": stage_summary(r, sparse),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": f"synthetic (seeded N(0,1) q/K/V, {cfg.tree} tree; {copies} rotated input copies)",
        "config": {"workload": wname, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.D, "context": cfg.L, "draft_nodes": cfg.N, "tree": cfg.tree,
                   "verify": "sparse" if sparse else "dense", "n_ctx_keys": n_ctx},
        "roofline": roof,
    }
    if sparse:
        line["gather_probe"], line["selector"] = sparse_extras(torch, ops, cfg, sets, r, es)
    if other is not None:
        # the same inputs verified in the workload's other mode, timed the same way
        print(f"[bench] timing the {'sparse' if other else 'dense'} mode", file=sys.stderr, flush=True)
        oname = workload_name(cfg, other)
        r2 = run_steps(torch, ops, cfg, other, sets, dev, args.steps, args.warmup)
        a2 = algorithmic(cfg, r2["n_ctx"], other)
        o = {"workload": oname, "verify": "sparse" if other else "dense", "n_ctx_keys": r2["n_ctx"],
             "ms_per_step": round(r2["ms_per_step"], 4),
             "gbs": round(a2["step_bytes"] / (r2["ms_per_step"] * 1e-3) / 1e9, 1),
             "draft_tokens_verified_per_s_per_layer": round(cfg.B * cfg.N / (r2["ms_per_step"] * 1e-3), 1),
             "speedup_vs_" + ("dense" if other else "sparse"):
                 round((ms_per_step / r2["ms_per_step"]) if other else (r2["ms_per_step"] / ms_per_step), 3),
             "stage_ms": stage_summary(r2, other),
             "roofline": roofline_of(cfg, other, r2, read_peak, oname)}
        if other:
            o["gather_probe"], o["selector"] = sparse_extras(torch, ops, cfg, sets, r2, es)
        line["sparse_step" if other else "dense_step"] = o
    line["accept_commit"] = measure_commit(torch, ops, cfg, x, base, dev)
    line["importance_scores"] = measure_scores(torch, ops, cfg, sets, dev, ms_per_step)
    line["draft_tree"] = measure_tree(torch, ops, cfg, dev)
    if args.copy_calib_gib > 0:
        n = int(args.copy_calib_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_budget, sparse)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
