"""GPU importance scores against the oracle (Dustin, "Metodologia" sections 1-2).

Tolerance: scores are sums of probabilities exp2(s - lse2) with s from bf16
inputs accumulated in fp32 and lse2 from fp32 sums over up to 2^17 tokens;
relative error ~1e-5, so rtol 1e-4 with a tiny absolute floor."""

import numpy as np
import pytest
import torch

from long_context_verify_tree_amd import synth
from oracle import verify_oracle as vo

from _util import to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _bf16(rng, *shape, scale=1.0):
    return synth.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


def _gpu(gpu_lib, q, k, scale=None, k_view=None):
    dq = to_dev(q, synth.BF16)
    dk = to_dev(k, synth.BF16) if k_view is None else k_view
    out = gpu_lib.importance_scores(dq, dk, scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("M,L", [(1, 1), (8, 31), (8, 600), (32, 5000), (5, 70001)])
def test_scores_match_oracle(gpu_lib, D, M, L):
    rng = np.random.default_rng(D * 1000 + M * 7 + L)
    B, Hs = 2, 3
    q, k = _bf16(rng, B, Hs, M, D), _bf16(rng, B, Hs, L, D)
    say(f"case scores D={D} M={M} L={L}")
    got = _gpu(gpu_lib, q, k)
    ref = vo.importance_scores(q, k)
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-9)
    np.testing.assert_allclose(got.sum(axis=1), Hs * M, rtol=1e-4)


def test_scores_peaky_and_scale(gpu_lib):
    # large logits: the max must be tracked across splits and wavefronts
    rng = np.random.default_rng(31)
    B, Hs, M, L, D = 2, 2, 8, 9000, 128
    q, k = _bf16(rng, B, Hs, M, D, scale=3.0), _bf16(rng, B, Hs, L, D, scale=3.0)
    say("case scores peaky")
    np.testing.assert_allclose(_gpu(gpu_lib, q, k), vo.importance_scores(q, k), rtol=1e-4, atol=1e-9)
    np.testing.assert_allclose(_gpu(gpu_lib, q, k, scale=0.01), vo.importance_scores(q, k, scale=0.01),
                               rtol=1e-4, atol=1e-9)


def test_scores_strided_heads(gpu_lib):
    # the scoring heads are every other head of a [B, 2 Hs, L, D] cache
    rng = np.random.default_rng(32)
    B, Hs, M, L, D = 3, 2, 8, 3000, 128
    cache = _bf16(rng, B, 2 * Hs, L, D)
    q = _bf16(rng, B, Hs, M, D)
    dk = to_dev(cache, synth.BF16)[:, ::2]
    say("case scores strided heads")
    np.testing.assert_allclose(_gpu(gpu_lib, q, None, k_view=dk), vo.importance_scores(q, cache[:, ::2]),
                               rtol=1e-4, atol=1e-9)


def test_scores_full_size_qwen_sparse_workload(gpu_lib):
    # the sparse Qwen2.5-7B workload's shape: 16 sequences, 32768 tokens, two
    # scoring heads with the 8 draft rows each
    cfg = synth.CONFIGS["qwen25_7b_sparse2048_L32k"]
    rng = np.random.default_rng(cfg.seed + 1)
    q, k = _bf16(rng, cfg.B, 2, cfg.N, cfg.D), _bf16(rng, cfg.B, 2, cfg.L, cfg.D)
    say("case scores full size")
    got = _gpu(gpu_lib, q, k)
    ref = vo.importance_scores(q, k)
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-9)
