"""Host-side logic of bench.py (no GPU): verify-mode selection, workload
names, which selector kernel a shape runs, algorithmic byte/flop counts and
the staleness rule of the committed rocprofv3 summaries."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_verify_tree_amd import synth  # noqa: E402

C = synth.CONFIGS


def test_verify_mode_and_names():
    assert bench.verify_mode(C["llama3_8b_chain8_L32k"], "auto") is False
    assert bench.verify_mode(C["qwen25_7b_sparse2048_L32k"], "auto") is True
    assert bench.verify_mode(C["l70b_tree128_L128k"], "auto") is False        # dense and sparse: dense by default
    assert bench.verify_mode(C["l70b_tree128_L128k"], "sparse") is True
    assert bench.verify_mode(C["qwen25_7b_sparse2048_L32k"], "dense") is False
    with pytest.raises(SystemExit):
        bench.verify_mode(C["llama3_8b_chain8_L32k"], "sparse")              # no verify-set parameters
    assert bench.workload_name(C["l70b_tree128_L128k"], False) == "l70b_tree128_L128k"
    assert bench.workload_name(C["l70b_tree128_L128k"], True) == "l70b_tree128_L128k_sparse4096"
    assert bench.workload_name(C["qwen25_7b_sparse2048_L32k"], True) == "qwen25_7b_sparse2048_L32k"
    assert bench.workload_name(C["qwen25_7b_sparse2048_L32k"], False) == "qwen25_7b_sparse2048_L32k_dense"


def test_selector_kernel_choice():
    # a selection: the filter over many workgroups per row, then the resolve
    assert bench.select_kernel_name(16, 32768, 2048) == "select_filter_kernel+select_resolve_kernel"
    assert bench.select_kernel_name(4, 131072, 4096) == "select_filter_kernel+select_resolve_kernel"
    # budget >= L: every index, written by the resolve kernel alone
    assert bench.select_kernel_name(4, 131072, 131072) == "select_resolve_kernel"


def test_algorithmic_counts():
    cfg = C["llama3_8b_chain8_L32k"]
    a = bench.algorithmic(cfg, cfg.L, False)
    assert a["kv"] == 2 * 8 * 8 * 32768 * 128 * 2
    assert a["partial_bytes"] == 1074528512                   # K/V + q + draft K/V + parent
    assert a["flops"] == 4 * 8 * 32 * 8 * 32768 * 128
    sp = C["qwen25_7b_sparse2048_L32k"]
    s = bench.algorithmic(sp, sp.budget, True)
    assert s["kv"] == 2 * 16 * 4 * 2048 * 128 * 2
    assert s["partial_bytes"] - s["kv"] == (16 * 28 * 8 * 128 * 2 + 2 * 16 * 4 * 8 * 128 * 2 + 16 * 2048 * 4
                                            + 16 * 8 * 4)


def test_committed_summaries_fresh_and_stale(tmp_path, monkeypatch):
    # the committed headline summary matches the current kernel source
    traffic, src = bench.committed_traffic("partial_kernel", "llama3_8b_chain8_L32k")
    assert traffic is not None and src.endswith("partial_kernel_llama3_8b_chain8_L32k.md")
    # a copy of the summary with another source hash reads as stale
    prof = tmp_path / "profiles"
    prof.mkdir()
    text = open(os.path.join(ROOT, "profiles", "partial_kernel_llama3_8b_chain8_L32k.md")).read()
    lines = [("- kernel source sha256: `" + "0" * 64 + "`") if l.startswith("- kernel source sha256") else l
             for l in text.splitlines()]
    (prof / "partial_kernel_llama3_8b_chain8_L32k.md").write_text("\n".join(lines))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    traffic, note = bench.committed_traffic("partial_kernel", "llama3_8b_chain8_L32k")
    assert traffic is None and "stale" in note
    assert bench.committed_traffic("partial_kernel", "no_such_workload") == (None, None)


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_more_than_one_gpu_is_refused():
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU only" in res.stderr


def test_committed_mfma_util():
    pct, src = bench.committed_mfma_util("rows_kernel", "l70b_tree128_L128k")
    assert src == "profiles/rows_kernel_l70b_tree128_L128k_pipes.md"
    assert pct is not None and 0.0 < pct < 100.0
    # no pipe summary for this kernel and workload
    assert bench.committed_mfma_util("select_kernel", "qwen25_7b_sparse2048_L32k") == (None, None)
