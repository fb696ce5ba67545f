"""Oracle: SnapKV/PyramidKV observation-window token selection.

Test infrastructure (see the package docstring).  Scores in float64.
"""

import numpy as np


def window_scores(q_win, k, W):
    """Attention mass each candidate prompt position receives from the window.

    Blog, "Eviction: keep fewer tokens" (SnapKV: look at the attention the last
    few prompt tokens pay to the rest, per head); PyramidKV Sec. "KV Cache
    Selection" (score of token i summed over the instruction tokens [n-alpha, n]
    of the attention of each head; the formulas themselves are missing from the
    page).  Readings: each window row is the model's own causal softmax row
    (keys 0..p_r, scaled by 1/sqrt(D)); the score of candidate c < n-W is the sum
    of the normalized probabilities over the W window rows and over the G query
    heads that share the KV head (repeat_kv grouping, blog attention hook).

    q_win: float [B][Hq][W][D] (values of the model dtype), k: float [B][Hkv][n][D].
    Returns float64 [B][Hkv][n-W].
    """
    q_win = np.asarray(q_win, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Wq, D = q_win.shape
    _, Hkv, n, _ = k.shape
    assert Wq == W and Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((B, Hkv, n - W), dtype=np.float64)
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for j in range(Hkv):
            for h in range(j * G, (j + 1) * G):
                for r in range(W):
                    p = n - W + r  # absolute position of this window query
                    logits = (k[b, j, : p + 1] @ q_win[b, h, r]) * scale
                    e = np.exp(logits - logits.max())
                    prob = e / e.sum()
                    out[b, j] += prob[: n - W]
    return out


def max_pool(s, pool):
    """1-D max pooling, kernel ``pool`` (odd), stride 1, same length, edges clipped.

    PyramidKV Sec. "KV Cache Selection" (a pooling layer over the attention, to
    avoid being misled by a few massive scores) and Sec. "Baselines" (SnapKV's
    clustering with a pooling layer).  Reading: max pooling, clipped window.
    """
    s = np.asarray(s)
    r = pool // 2
    N = s.shape[-1]
    out = np.empty_like(s)
    for c in range(N):
        lo, hi = max(0, c - r), min(N, c + r + 1)
        out[..., c] = s[..., lo:hi].max(axis=-1)
    return out


def top_k(scores, k):
    """Positions of the k' = min(k, N) largest scores, ascending.

    PyramidKV Sec. "KV Cache Selection": per layer and head the top k^l tokens
    by score are kept and the rest discarded.  Ties go to the lower index; the
    output is in ascending position order (kept tokens keep their positions).
    scores: 1-D array (any float dtype, compared exactly).
    """
    N = len(scores)
    kk = min(int(k), N)
    order = sorted(range(N), key=lambda c: (-float(scores[c]), c))
    return np.array(sorted(order[:kk]), dtype=np.int32)


def score_variance(scores):
    """Variance of the cumulated attention of each (b, KV head).

    MiniKV, Sec. 4.2 and the caption of Fig. 7: the variance score of a layer is
    Var(A_cumul), the variance of the cumulated attention map.  Readings: A_cumul
    of a KV head is its window column sums over the n - W candidates (the scores
    before pooling), and Var is the population variance over those positions;
    a layer's score is the mean of these over batch rows and KV heads (done by
    the caller).  scores: [..., N]; returns float64 [...].
    """
    s = np.asarray(scores, dtype=np.float64)
    mu = s.mean(axis=-1, keepdims=True)
    return ((s - mu) ** 2).mean(axis=-1)


def recent_select(n, W, budget, sinks):
    """Position-only selection: a few leading "sink" tokens plus the most recent.

    Blog, "Eviction: keep fewer tokens": a sliding window keeps only the last
    tokens; StreamingLLM keeps the first four tokens (attention sinks) as well.
    PyramidKV Sec. "Baselines": StreamingLLM keeps the first k - alpha and the
    last alpha tokens of the budget k.  Reading: as for the score-based
    selection, the observation window [n-W, n) is always kept and the budget
    k' = min(budget, n-W) (budget < 0: every candidate) counts the other prompt
    positions; the first s = min(sinks, k') positions are sinks and the last
    k' - s candidates are the recent part.  sinks = 0 is the sliding window of
    k' + W tokens.  Returns int32 [k'], ascending.
    """
    N = n - W
    kk = N if budget < 0 else min(budget, N)
    s = min(sinks, kk)
    first = list(range(s))
    recent = list(range(N - (kk - s), N))
    return np.array(first + recent, dtype=np.int32)


def select(q_win, k, W, pool, budget):
    """Full selection: window scores -> max pool -> per-(b, KV head) top-k.

    Returns (idx int32 [B][Hkv][k'], pooled float64 [B][Hkv][n-W]).
    """
    s = window_scores(q_win, k, W)
    sp = max_pool(s, pool)
    B, Hkv, N = sp.shape
    kk = min(budget, N) if budget >= 0 else N
    idx = np.zeros((B, Hkv, kk), dtype=np.int32)
    for b in range(B):
        for j in range(Hkv):
            idx[b, j] = top_k(sp[b, j], kk)
    return idx, sp
