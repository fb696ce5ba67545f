"""Helpers for the GPU parity tests: tensor <-> oracle conversions and the
comparison rules (bit-exact for codes, scales and indices; 2e-3 for outputs)."""

import numpy as np
import torch

from oracle import quant, select

DECODE_TOL = 2e-3   # max |o_gpu - o_ref| <= 2e-3 * max(1, max |o_ref|)
SCORE_TOL = 1e-5    # |s_gpu - s_ref| <= 1e-5 * (|s_ref| + max s_ref)


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def as_f32(t):
    """Model-dtype tensor -> float32 numpy (exact)."""
    return t.detach().float().cpu().numpy()


def bf16_bits(t):
    """Model-dtype tensor -> bf16 bits the residual stores (RNE from fp32)."""
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return quant.bf16_bits(t.detach().cpu().numpy())


def u32(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


def u16(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint16)


def gpu_head_cache(cache, b, j):
    v = cache.views()
    return {
        "q_len": cache.q_len, "r_len": cache.r_len,
        "k_codes": u32(v["k_codes"][b, j]), "k_meta": u32(v["k_meta"][b, j]),
        "v_codes": u32(v["v_codes"][b, j]), "v_meta": u32(v["v_meta"][b, j]),
        "k_res": u16(v["k_res"][b, j]), "v_res": u16(v["v_res"][b, j]),
    }


def gpu_all_caches(cache):
    """Every unit's logical cache state, copied to the host once: a dict of numpy
    arrays [B][Hkv][...] plus q_len / r_len (for unit_cache)."""
    v = cache.views()
    out = {"q_len": cache.q_len, "r_len": cache.r_len}
    for key in ("k_codes", "k_meta", "v_codes", "v_meta"):
        out[key] = u32(v[key])
    for key in ("k_res", "v_res"):
        out[key] = u16(v[key])
    return out


def unit_cache(allc, b, j):
    """One unit's cache from gpu_all_caches, in the layout of gpu_head_cache."""
    d = {"q_len": allc["q_len"], "r_len": allc["r_len"]}
    for key in ("k_codes", "k_meta", "v_codes", "v_meta", "k_res", "v_res"):
        d[key] = allc[key][b, j]
    return d


def assert_cache_equal(gpu, ref, where=""):
    assert gpu["q_len"] == ref["q_len"] and gpu["r_len"] == ref["r_len"], where
    for key in ("k_codes", "k_meta", "v_codes", "v_meta", "k_res", "v_res"):
        g, r = gpu[key], ref[key]
        assert g.shape == r.shape, (where, key, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{where} {key}: {len(bad)} mismatches, first at {bad[0].tolist()}: "
                                 f"gpu {g[tuple(bad[0])]:#x} ref {r[tuple(bad[0])]:#x}")


def assert_decode_close(out_gpu, out_ref, where=""):
    err = np.max(np.abs(out_gpu.astype(np.float64) - out_ref))
    lim = DECODE_TOL * max(1.0, float(np.max(np.abs(out_ref))))
    assert err <= lim, f"{where}: max abs err {err:.3e} > {lim:.3e}"
    return err


def check_selection(idx_gpu, scores_gpu, pooled_ref, budget):
    """P-S1 scores close, P-S3a idx exact on the GPU's own scores, P-S3b same set
    as the oracle's up to swaps among near-ties of the k'-th score.  Returns the
    number of near-tie swaps."""
    N = pooled_ref.shape[-1]
    kk = N if budget < 0 else min(budget, N)
    assert idx_gpu.shape[-1] == kk
    smax = pooled_ref.max()
    np.testing.assert_array_less(np.abs(scores_gpu - pooled_ref), SCORE_TOL * (np.abs(pooled_ref) + smax) + 1e-30)
    exact = select.top_k(scores_gpu, kk)
    np.testing.assert_array_equal(idx_gpu, exact)
    ref = select.top_k(pooled_ref, kk)
    diff = set(idx_gpu.tolist()) ^ set(ref.tolist())
    if diff and kk > 0:
        kth = np.sort(pooled_ref)[::-1][kk - 1]
        for c in diff:
            assert abs(pooled_ref[c] - kth) <= SCORE_TOL * (abs(kth) + smax), (c, pooled_ref[c], kth)
    return len(diff) // 2
