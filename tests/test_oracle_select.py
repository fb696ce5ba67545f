"""Pins of the oracle's selection (window scores, max pool, top-k) against a
library softmax, brute force on tiny inputs and the invariants of the method."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import select


def _case(seed, B, Hq, Hkv, n, W, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, W, D))
    k = rng.standard_normal((B, Hkv, n, D)) * rng.lognormal(0, 0.5, size=(1, Hkv, 1, D))
    return q, k


@pytest.mark.parametrize("B,Hq,Hkv,n,W,D", [(1, 4, 4, 40, 8, 16), (2, 8, 2, 67, 5, 32),
                                            (1, 2, 1, 9, 9, 8)])
def test_scores_match_torch_causal_softmax(B, Hq, Hkv, n, W, D):
    q, k = _case(1, B, Hq, Hkv, n, W, D)
    got = select.window_scores(q, k, W)
    G = Hq // Hkv
    qt = torch.tensor(q)
    kt = torch.tensor(k).repeat_interleave(G, dim=1)            # [B][Hq][n][D]
    logits = qt @ kt.transpose(-1, -2) / math.sqrt(D)           # [B][Hq][W][n]
    pos = torch.arange(n - W, n)[:, None]
    mask = torch.arange(n)[None, :] > pos                       # causal rows of the window
    P = torch.softmax(logits.masked_fill(mask, float("-inf")), dim=-1)
    ref = P.sum(dim=2).view(B, Hkv, G, n).sum(dim=2)[..., : n - W]
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)
    # every window row sums to one: candidates + window mass = W*G per KV head
    win = P.sum(dim=2).view(B, Hkv, G, n).sum(dim=2)[..., n - W:]
    np.testing.assert_allclose(got.sum(-1) + win.sum(-1).numpy(), W * G, rtol=1e-12)


def test_scores_brute_force_python_loops():
    q, k = _case(2, 1, 2, 1, 7, 3, 4)
    got = select.window_scores(q, k, 3)
    n, W, D = 7, 3, 4
    ref = [0.0] * (n - W)
    for h in range(2):
        for r in range(W):
            p = n - W + r
            ls = [sum(q[0, h, r, d] * k[0, 0, c, d] for d in range(D)) / math.sqrt(D)
                  for c in range(p + 1)]
            z = sum(math.exp(v) for v in ls)
            for c in range(n - W):
                ref[c] += math.exp(ls[c]) / z
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-12)


@pytest.mark.parametrize("pool", [1, 3, 5, 7])
def test_max_pool_matches_torch(pool):
    rng = np.random.default_rng(pool)
    s = rng.random((2, 3, 50))
    got = select.max_pool(s, pool)
    ref = torch.nn.functional.max_pool1d(torch.tensor(s), pool, stride=1, padding=pool // 2)
    np.testing.assert_array_equal(got, ref.numpy())
    if pool == 1:
        np.testing.assert_array_equal(got, s)


def _rank_select(s, k):
    """Independent formulation: c is kept iff fewer than k candidates beat it."""
    N = len(s)
    keep = []
    for c in range(N):
        beat = sum(1 for d in range(N) if s[d] > s[c] or (s[d] == s[c] and d < c))
        if beat < k:
            keep.append(c)
    return keep


@pytest.mark.parametrize("seed", range(6))
def test_top_k_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    N = 13
    s = rng.integers(0, 4, N).astype(np.float32)   # many exact ties
    for k in [0, 1, 3, 7, 12, 13, 20]:
        got = list(select.top_k(s, k))
        assert got == _rank_select(s, min(k, N))
        assert got == sorted(got)
        # optimality: no unselected score exceeds a selected one
        if 0 < len(got) < N:
            rest = [c for c in range(N) if c not in got]
            assert min(s[got]) >= max(s[rest])


def test_top_k_exhaustive_tiny():
    # brute force over all subsets: the kept set maximizes the score sum, then is
    # lexicographically smallest among maximizers
    s = np.array([0.5, 0.25, 0.5, 0.75, 0.25, 0.5], dtype=np.float32)
    for k in range(0, 7):
        best = max(itertools.combinations(range(6), k),
                   key=lambda c: (sum(s[list(c)]), [-i for i in c]))
        assert list(select.top_k(s, k)) == list(best)


def test_select_budget_covers_everything():
    q, k = _case(3, 1, 4, 2, 30, 6, 8)
    idx, _ = select.select(q, k, 6, 3, 1000)
    assert idx.shape == (1, 2, 24)
    np.testing.assert_array_equal(idx[0, 0], np.arange(24))


def test_planted_heavy_tokens_are_found():
    # sanity (not parity): keys aligned with the window queries win the selection
    rng = np.random.default_rng(7)
    D, n, W = 32, 200, 8
    q = rng.standard_normal((1, 2, W, D))
    k = rng.standard_normal((1, 1, n, D))
    mu = q.reshape(-1, D).mean(0)
    mu /= np.linalg.norm(mu)
    heavy = rng.choice(np.arange(4, n - W), 10, replace=False)
    k[0, 0, heavy] += 6 * math.sqrt(D) * mu
    idx, _ = select.select(q, k, W, 1, 10)
    assert set(idx[0, 0].tolist()) == set(heavy.tolist())


# ---- variance of the cumulated attention (MiniKV Sec. 4.2, Fig. 7)

def test_score_variance_closed_forms():
    assert select.score_variance(np.full(17, 3.25)) == 0.0
    assert select.score_variance(np.array([1.0, 2.0, 3.0, 4.0])) == 1.25
    # 0..N-1: (N^2 - 1) / 12
    for N in (1, 2, 7, 100):
        assert math.isclose(select.score_variance(np.arange(N, dtype=np.float64)), (N * N - 1) / 12.0,
                            rel_tol=1e-12, abs_tol=1e-15)


def test_score_variance_batched_and_shift_invariant():
    rng = np.random.default_rng(3)
    s = rng.random((2, 3, 50))
    v = select.score_variance(s)
    assert v.shape == (2, 3)
    np.testing.assert_allclose(select.score_variance(s + 7.0), v, rtol=1e-9)
    np.testing.assert_allclose(select.score_variance(4.0 * s), 16.0 * v, rtol=1e-12)
    # a single outlier of height h on N zeros: h^2 (N-1) / N^2
    z = np.zeros(40)
    z[5] = 3.0
    assert math.isclose(select.score_variance(z), 9.0 * 39 / 1600, rel_tol=1e-12)


# ---------------------------------------------------------------- sinks + window
@pytest.mark.parametrize("sinks,cache", [(4, 512), (0, 256), (4, 256), (0, 128), (4, 128)])
def test_recent_select_blog_table_configurations(sinks, cache):
    """Blog, "Eviction" measurements: caches of "4 sink tokens + the last 508",
    "the last 256 tokens", "4 sink tokens + the last 252", ...  With the window
    kept as always, the whole cache is the first `sinks` prompt tokens plus the
    last cache - sinks."""
    from oracle import quant
    n = 4096
    for W in (1, 8, 32):
        idx = select.recent_select(n, W, cache - W, sinks)
        kept = quant.kept_positions(n, W, idx)
        assert len(kept) == cache
        assert list(kept) == list(range(sinks)) + list(range(n - (cache - sinks), n))


def test_recent_select_pyramidkv_baseline_split():
    """PyramidKV "Baselines": StreamingLLM keeps the first k - alpha and the last
    alpha tokens of a budget k."""
    n, W = 1000, 10
    for k, alpha in ((100, 60), (64, 64), (64, 0), (7, 3)):
        idx = select.recent_select(n, W, k, k - alpha)
        assert list(idx[: k - alpha]) == list(range(k - alpha))
        assert list(idx[k - alpha:]) == list(range(n - W - alpha, n - W))


def test_recent_select_is_top_k_of_a_position_priority():
    """Every tiny case: the selection equals the top-k' candidates when sinks
    rank first and the others rank by position (a different route through the
    same definition)."""
    for n in range(1, 12):
        for W in range(1, n + 1):
            N = n - W
            for budget in range(-1, N + 2):
                for sinks in range(0, N + 2):
                    kk = N if budget < 0 else min(budget, N)
                    pri = np.array([np.inf if c < sinks else float(c) for c in range(N)])
                    want = select.top_k(pri, kk) if N else np.zeros(0, np.int32)
                    got = select.recent_select(n, W, budget, sinks)
                    assert got.dtype == np.int32 and list(got) == list(want), (n, W, budget, sinks)


def test_recent_select_degenerate():
    assert list(select.recent_select(50, 10, 0, 4)) == []
    assert list(select.recent_select(50, 50, 5, 4)) == []
    assert list(select.recent_select(50, 10, 100, 4)) == list(range(40))
    assert list(select.recent_select(50, 10, -1, 0)) == list(range(40))
    assert list(select.recent_select(50, 10, 3, 9)) == [0, 1, 2]
