"""GPU parity of the verify-set selector's two ways of finding a tier's
threshold (Dustin, "Aggregazione Ibrida dell'Attenzione"): the short way
(sampled window, one sweep, a list resolved by a finer histogram and a
pairwise comparison) and the exact radix way, which the test hook
VA_SELECT_EXACT=1 forces.  Both must return the oracle's index list bit for
bit, on rows of one to many filter segments, with and without a small group
of equal scores at each tier's threshold.
Expected values come only from ``oracle``."""

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo

pytestmark = pytest.mark.gpu

# (B, L, sink, window, top_m, budget): the Qwen2.5-7B and 70B-shape sparse
# workloads, a short row, and rows of 3 and 5 multi-workgroup segments
SHAPES = [
    (16, 32768, 4, 256, 1024, 2048),
    (4, 131072, 4, 256, 2048, 4096),
    (3, 5000, 4, 16, 300, 900),
    (1, 40000, 4, 256, 1500, 3000),
    (2, 70001, 4, 256, 1024, 2048),
]


def say(*a):
    print(*a, flush=True)


def _sel(ops, d, t, sink, window, m, budget):
    g = ops.select_verify_set(torch.from_numpy(d).cuda(), torch.from_numpy(t).cuda(), sink=sink, window=window,
                              top_m=m, budget=budget)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def _plant_ties(rng, d, t, sink, window, m, budget, n=20):
    """Give n more free tokens of each row the score of that tier's last
    pick, so that each threshold falls inside a group of about n + 1 equal
    scores (the oracle's lower-index rule then decides)."""
    B, L = d.shape
    prot = vo.protected_set(L, sink, window)
    free = np.setdiff1d(np.arange(L), prot)
    rest = budget - len(prot)
    r1 = min(m, rest, len(free))
    r2 = rest - r1
    for b in range(B):
        if r1 > 0:
            v = np.sort(d[b, free])[::-1][r1 - 1]
            d[b, rng.choice(free, n, replace=False)] = v
        if r2 > 0:
            dset = vo.select_verify_set(d[b:b + 1], t[b:b + 1], sink, window, r1, len(prot) + r1)[0]
            remain = np.setdiff1d(free, dset)
            v = np.sort(t[b, remain])[::-1][r2 - 1]
            t[b, rng.choice(remain, n, replace=False)] = v
    return d, t


@pytest.mark.parametrize("exact", [False, True], ids=["short", "exact"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_L{s[1]}")
def test_both_ways_match_the_oracle(gpu_lib, monkeypatch, shape, exact):
    B, L, S, W, m, budget = shape
    if exact:
        monkeypatch.setenv("VA_SELECT_EXACT", "1")
    rng = np.random.default_rng(L + B)
    d = rng.lognormal(0, 2, (B, L)).astype(np.float32)
    t = rng.lognormal(0, 2, (B, L)).astype(np.float32)
    say(f"case selector {'exact' if exact else 'short'} way B={B} L={L} budget={budget}")
    got = _sel(gpu_lib, d, t, S, W, m, budget)
    np.testing.assert_array_equal(got, vo.select_verify_set(d, t, S, W, m, budget))


@pytest.mark.parametrize("exact", [False, True], ids=["short", "exact"])
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[1], SHAPES[2], SHAPES[4]], ids=lambda s: f"B{s[0]}_L{s[1]}")
def test_small_tie_groups_at_the_thresholds(gpu_lib, monkeypatch, shape, exact):
    B, L, S, W, m, budget = shape
    B = min(B, 4)
    if exact:
        monkeypatch.setenv("VA_SELECT_EXACT", "1")
    rng = np.random.default_rng(7 * L + B)
    d = rng.lognormal(0, 2, (B, L)).astype(np.float32)
    t = rng.lognormal(0, 2, (B, L)).astype(np.float32)
    d, t = _plant_ties(rng, d, t, S, W, m, budget)
    say(f"case selector ties at the thresholds, {'exact' if exact else 'short'} way B={B} L={L}")
    got = _sel(gpu_lib, d, t, S, W, m, budget)
    np.testing.assert_array_equal(got, vo.select_verify_set(d, t, S, W, m, budget))


def test_sample_far_from_the_threshold(gpu_lib):
    # Scores rising along the row: the top tokens sit at the end, the window
    # of a one-in-eight sample is narrow, and large budgets put the threshold
    # near the bottom of the candidates.  Every budget must still give the
    # oracle's list, whichever way finds it.
    L = 32768
    d = np.linspace(1.0, 2.0, L, dtype=np.float32)[None].repeat(2, 0)
    t = np.linspace(2.0, 1.0, L, dtype=np.float32)[None].repeat(2, 0)
    d[1] = d[1][::-1]
    for (m, budget) in ((10, 300), (5000, 20000), (20000, 30000), (1, 261)):
        say(f"case selector monotone scores m={m} budget={budget}")
        got = _sel(gpu_lib, d, t, 4, 256, m, budget)
        np.testing.assert_array_equal(got, vo.select_verify_set(d, t, 4, 256, m, budget))
