"""Oracle: prefill attention that also returns the attention each key position
accumulates, heavy-hitter (H2O) selection on it, and its variance score.

Test infrastructure (see the package docstring).  Attention in float64.

Sources:
  * MiniKV Sec. 4.3 "Selective KV Compatible Attention Kernels" and Fig. 9:
    a FlashAttention-style prefill that returns, besides the attention output,
    the attention accumulated along each key column (A_cumul), at O(l_key) extra
    memory.  The page's kernel leaves out each row's normalization (it would
    need the whole row).  Reading used here: A_cumul is the column sum of the
    *normalized* causal attention probabilities, i.e. the accumulated attention
    of H2O; the per-row log-sum-exp that normalization needs is O(l_query)
    numbers, which a FlashAttention forward produces anyway.  With it the
    result is independent of tile sizes and processing order.
  * Blog "Eviction: keep fewer tokens" (heavy hitters: keep the tokens with the
    largest accumulated attention plus a recent window) and PyramidKV
    "Baselines" (H2O ranks tokens by the attention all queries pay them).
  * MiniKV Sec. 4.2 and the caption of Fig. 7: the variance score Var(A_cumul).
"""

import numpy as np

from . import select


def attention_colsums(q, k, v, row_from=0, row_block=1024):
    """Causal GQA attention of every prompt row, and the column sums of its
    probabilities.

    For query head h (KV head j = h // G, repeat_kv grouping as in the blog's
    attention hook) and row r, P_r = softmax over keys c <= r of
    q_r . k_c / sqrt(D) (MiniKV Eq. 1 for one query; causal prefill), and
    O[h, r] = sum_c P_rc v_c.  A_cumul[j, c] = sum over the G heads of KV head j
    and over rows r >= row_from of P_rc (MiniKV Sec. 4.3; the reading in the
    module docstring: normalized probabilities).

    q: float [B][Hq][n][D]; k, v: float [B][Hkv][n][D] (values of the model
    dtype).  Rows are processed in blocks of row_block (memory only; the
    arithmetic per row is the same).  Returns (O float64 [B][Hq][n][D],
    A_cumul float64 [B][Hkv][n]); O rows below row_from are zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0 and k.shape == (B, Hkv, n, D) and v.shape == k.shape
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    O = np.zeros((B, Hq, n, D), dtype=np.float64)
    acc = np.zeros((B, Hkv, n), dtype=np.float64)
    cols = np.arange(n)
    for b in range(B):
        for h in range(Hq):
            j = h // G
            for r0 in range(row_from, n, row_block):
                r1 = min(n, r0 + row_block)
                logits = (q[b, h, r0:r1] @ k[b, j].T) * scale          # [rows][n]
                logits[cols[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
                e = np.exp(logits - logits.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                O[b, h, r0:r1] = p @ v[b, j]
                acc[b, j] += p.sum(axis=0)
    return O, acc


def row_lse(q, k):
    """Each prompt row's log-sum-exp (natural log) of its causal logits
    q_r . k_c / sqrt(D) over c <= r: the softmax normalizer the prefill's
    FlashAttention keeps (MiniKV Sec. 4.3), which normalizes each row of
    attention_colsums.  q [B][Hq][n][D], k [B][Hkv][n][D]; returns float64
    [B][Hq][n]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, n, D = q.shape
    G = Hq // k.shape[1]
    out = np.empty((B, Hq, n))
    mask = np.arange(n)[None, :] > np.arange(n)[:, None]
    for b in range(B):
        for h in range(Hq):
            x = (q[b, h] @ k[b, h // G].T) / np.sqrt(D)
            x[mask] = -np.inf
            m = x.max(axis=1)
            out[b, h] = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    return out


def h2o_select(acc_row, n, W, budget):
    """Heavy hitters plus the recent window for one (b, KV head).

    Blog "Eviction: keep fewer tokens": H2O keeps the tokens with the largest
    accumulated attention plus a recent window.  As for the window-scored
    selection, the last W positions are always kept and the budget
    k' = min(budget, n - W) (budget < 0: all) counts the other candidates
    [0, n - W), taken by accumulated attention with ties to the lower position,
    ascending.  No pooling (H2O ranks single tokens).
    """
    N = n - W
    kk = N if budget < 0 else min(budget, N)
    return select.top_k(np.asarray(acc_row)[:N], kk)


def acc_variance(acc):
    """Var(A_cumul) over all n key positions of each (b, KV head), population
    variance (MiniKV Sec. 4.2 and Fig. 7, with A_cumul over every query row)."""
    return select.score_variance(acc)
