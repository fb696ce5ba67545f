"""Oracle: single-query decode attention over the compressed cache.

Test infrastructure (see the package docstring).  Attention in float64.
"""

import numpy as np

from . import quant


def head_keys_values(cache, bits):
    """Keys and values the decode step attends to, float64 [Q+r][D].

    The packed history is dequantized in float32 (zero + code*scale), then the
    bf16 residual follows, oldest first (MiniKV Alg. 1: concatenation of the
    dequantized history and the residual R_K, R_V).
    """
    g = cache.get("group", quant.GROUP)
    Kq = quant.unpack_keys(cache["k_codes"], cache["k_meta"], bits, g)
    Vq = quant.unpack_values(cache["v_codes"], cache["v_meta"], bits, g)
    Kr = quant.bf16_to_f32(cache["k_res"])
    Vr = quant.bf16_to_f32(cache["v_res"])
    K = np.concatenate([Kq, Kr], axis=0).astype(np.float64)
    V = np.concatenate([Vq, Vr], axis=0).astype(np.float64)
    return K, V


def attend(q, K, V):
    """softmax(q K^T / sqrt(D)) V for one query head (MiniKV Eq. 1), float64."""
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    logits = (K @ q) / np.sqrt(D)
    e = np.exp(logits - logits.max())
    p = e / e.sum()
    return p @ V


def decode_step(caches, q, k_new_bits, v_new_bits, residual, bits):
    """One decode step for one batch row.

    MiniKV Alg. 1 decoding: append the new key/value to the residual, flush it
    into the packed history when full, then one softmax over the concatenation
    of history scores and residual scores and the weighted sum of dequantized
    history values plus residual values.  Blog ``attention()`` hook: the same
    single softmax over full-precision recent tokens and rounded older ones;
    query head h reads KV head floor(h/G) (repeat_kv).

    caches: list over KV heads of per-head cache dicts (``quant`` layout).
    q: float [Hq][D] (model-dtype values); k_new_bits, v_new_bits: bf16 bits
    [Hkv][D].  Returns (out float64 [Hq][D], updated caches).
    """
    Hkv = len(caches)
    Hq = q.shape[0]
    G = Hq // Hkv
    new = [quant.append_and_flush(caches[j], k_new_bits[j], v_new_bits[j], residual, bits)
           for j in range(Hkv)]
    out = np.zeros(q.shape, dtype=np.float64)
    for j in range(Hkv):
        K, V = head_keys_values(new[j], bits)
        for h in range(j * G, (j + 1) * G):
            out[h] = attend(q[h], K, V)
    return out, new
