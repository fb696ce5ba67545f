"""Pins of oracle.prefill (MiniKV Sec. 4.3, selective flash-attention: the
prefill output plus the attention accumulated by each key column; H2O selection
on it; Var(A_cumul)).  Each check rests on something other than the oracle
itself: a library routine, brute force, a closed form or an invariant."""

import math

import numpy as np
import pytest
import torch

from oracle import prefill, select


def _case(seed, B, Hq, Hkv, n, D, key_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, n, D))
    k = rng.standard_normal((B, Hkv, n, D)) * key_scale
    v = rng.standard_normal((B, Hkv, n, D))
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,n,D,blk", [(1, 4, 4, 37, 16, 1024), (2, 8, 2, 50, 32, 7),
                                              (1, 3, 1, 64, 8, 64), (1, 2, 2, 1, 4, 1024)])
def test_output_equals_torch_sdpa(B, Hq, Hkv, n, D, blk):
    """O against torch's scaled_dot_product_attention (causal, float64), with the
    KV heads repeated over their query groups; row blocking does not matter."""
    q, k, v = _case(1, B, Hq, Hkv, n, D, key_scale=2.0)
    O, _ = prefill.attention_colsums(q, k, v, row_block=blk)
    G = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, is_causal=True)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_colsums_brute_force():
    """A_cumul by plain Python loops with math.exp: every row's causal softmax,
    summed per column over the rows and the two heads of the group."""
    q, k, v = _case(2, 1, 4, 2, 7, 3)
    O, acc = prefill.attention_colsums(q, k, v)
    n, D, G = 7, 3, 2
    for j in range(2):
        ref = [0.0] * n
        for h in range(j * G, (j + 1) * G):
            for r in range(n):
                logits = [sum(q[0, h, r, d] * k[0, j, c, d] for d in range(D)) / math.sqrt(D) for c in range(r + 1)]
                mx = max(logits)
                e = [math.exp(x - mx) for x in logits]
                s = sum(e)
                for c in range(r + 1):
                    ref[c] += e[c] / s
                # the output row too, from the same probabilities
                o = [sum(e[c] / s * v[0, j, c, d] for c in range(r + 1)) for d in range(D)]
                np.testing.assert_allclose(O[0, h, r], o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(acc[0, j], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("G,n", [(1, 1), (4, 33), (2, 200)])
def test_row_mass_invariant(G, n):
    """Each row's probabilities sum to one, so a KV head's columns sum to G*n."""
    q, k, v = _case(3, 2, 2 * G, 2, n, 16, key_scale=3.0)
    _, acc = prefill.attention_colsums(q, k, v)
    np.testing.assert_allclose(acc.sum(axis=-1), G * n, rtol=1e-12)
    assert np.all(acc >= 0)


def test_equal_keys_give_harmonic_sums():
    """With every key equal each row attends uniformly to its r+1 keys, so
    column c receives G * sum_{r>=c} 1/(r+1) and every output row is the mean
    of the values so far."""
    n, D, G = 40, 8, 3
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, G, n, D))
    k = np.tile(rng.standard_normal(D), (1, 1, n, 1))
    v = rng.standard_normal((1, 1, n, D))
    O, acc = prefill.attention_colsums(q, k, v)
    harm = np.array([sum(1.0 / (r + 1) for r in range(c, n)) for c in range(n)])
    np.testing.assert_allclose(acc[0, 0], G * harm, rtol=1e-12)
    means = np.cumsum(v[0, 0], axis=0) / np.arange(1, n + 1)[:, None]
    for h in range(G):
        np.testing.assert_allclose(O[0, h], means, rtol=1e-11, atol=1e-13)


def test_first_row_attends_only_to_itself():
    q, k, v = _case(5, 1, 2, 1, 20, 8, key_scale=5.0)
    O, acc = prefill.attention_colsums(q, k, v)
    np.testing.assert_allclose(O[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0), rtol=1e-14)
    # the last key is seen by the last row only, once per head
    assert acc[0, 0, -1] > 0 and acc[0, 0, -1] <= 2.0


@pytest.mark.parametrize("W", [1, 8, 30])
def test_last_rows_equal_window_scores(W):
    """Summing only the last W rows gives the observation-window scores of the
    SnapKV path (select.window_scores, pinned to torch's softmax) on the
    candidates [0, n-W)."""
    q, k, v = _case(6, 1, 8, 2, 90, 16, key_scale=2.0)
    _, acc = prefill.attention_colsums(q, k, v, row_from=90 - W)
    ref = select.window_scores(q[:, :, 90 - W:], k, W)
    np.testing.assert_allclose(acc[:, :, :90 - W], ref, rtol=1e-12, atol=1e-15)


def test_h2o_select_rules():
    """Heavy hitters among [0, n-W), ties to the lower position, ascending; a
    budget of all candidates (or < 0) keeps everything; zero keeps nothing."""
    acc = np.array([0.5, 3.0, 3.0, 0.1, 2.0, 1.0, 9.0, 9.0])
    n, W = 8, 2
    assert prefill.h2o_select(acc, n, W, 2).tolist() == [1, 2]     # 9.0s are the window
    assert prefill.h2o_select(acc, n, W, 3).tolist() == [1, 2, 4]
    assert prefill.h2o_select(acc, n, W, 1).tolist() == [1]        # tie: lower position
    assert prefill.h2o_select(acc, n, W, 6).tolist() == list(range(6))
    assert prefill.h2o_select(acc, n, W, -1).tolist() == list(range(6))
    assert prefill.h2o_select(acc, n, W, 0).tolist() == []
    # brute force on random rows against a full stable sort
    rng = np.random.default_rng(7)
    for _ in range(20):
        a = rng.integers(0, 5, 30).astype(np.float64)
        kk = int(rng.integers(0, 30))
        order = sorted(range(26), key=lambda c: (-a[c], c))[:kk]
        assert prefill.h2o_select(a, 30, 4, kk).tolist() == sorted(order)


def test_variance_closed_forms():
    """Var(A_cumul) over the n positions: zero for constant columns; for the
    equal-keys case, the population variance of G times the harmonic tails."""
    assert prefill.acc_variance(np.full((1, 1, 9), 2.5))[0, 0] == 0.0
    n, G = 25, 2
    harm = np.array([G * sum(1.0 / (r + 1) for r in range(c, n)) for c in range(n)])
    mu = sum(harm) / n
    ref = sum((x - mu) ** 2 for x in harm) / n
    assert prefill.acc_variance(harm[None, None])[0, 0] == pytest.approx(ref, rel=1e-12)


def test_row_lse_brute_force_and_bounds():
    """row_lse by plain loops with math.exp on a tiny case; in general
    max_c x_rc <= lse_r <= max_c x_rc + log(r + 1), and with equal keys
    lse_r = x + log(r + 1) exactly."""
    q, k, _ = _case(9, 1, 4, 2, 9, 5)
    lse = prefill.row_lse(q, k)
    for h in range(4):
        for r in range(9):
            xs = [sum(q[0, h, r, d] * k[0, h // 2, c, d] for d in range(5)) / math.sqrt(5) for c in range(r + 1)]
            assert lse[0, h, r] == pytest.approx(math.log(sum(math.exp(x) for x in xs)), rel=1e-12, abs=1e-12)
    q, k, _ = _case(10, 2, 4, 2, 60, 16, key_scale=3.0)
    lse = prefill.row_lse(q, k)
    x = np.einsum("bhrd,bjcd->bhjrc", q, k)  # every head against every KV head; take its own below
    for h in range(4):
        xs = x[:, h, h // 2] / 4.0
        xs = np.where(np.arange(60)[None, None, :] > np.arange(60)[None, :, None], -np.inf, xs)
        mx = xs.max(axis=-1)
        assert np.all(lse[:, h] >= mx - 1e-12) and np.all(lse[:, h] <= mx + np.log(np.arange(1, 61)) + 1e-12)
    n, D = 20, 8
    rng = np.random.default_rng(11)
    kk = np.tile(rng.standard_normal(D), (1, 1, n, 1))
    qq = rng.standard_normal((1, 2, n, D))
    lse = prefill.row_lse(qq, kk)
    xv = (qq[0] @ kk[0, 0, 0]) / np.sqrt(D)
    np.testing.assert_allclose(lse[0], xv + np.log(np.arange(1, n + 1))[None, :], rtol=1e-13, atol=1e-13)


def test_colsums_normalized_by_row_lse():
    """attention_colsums' probabilities are exp(x - row_lse): rebuilding A_cumul
    from row_lse gives the same columns."""
    q, k, v = _case(12, 1, 4, 2, 40, 8, key_scale=2.0)
    _, acc = prefill.attention_colsums(q, k, v)
    lse = prefill.row_lse(q, k)
    n, G = 40, 2
    ref = np.zeros((1, 2, n))
    for h in range(4):
        x = (q[0, h] @ k[0, h // G].T) / np.sqrt(8)
        x[np.arange(n)[None, :] > np.arange(n)[:, None]] = -np.inf
        ref[0, h // G] += np.exp(x - lse[0, h][:, None]).sum(axis=0)
    np.testing.assert_allclose(acc, ref, rtol=1e-12)
