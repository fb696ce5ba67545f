"""Pins of the oracle's cache builder, residual flush and decode attention
against torch SDPA, the dense special case, the blog's masked attention hook and
the equivalence of incremental flushes with batch quantization."""

import math

import numpy as np
import pytest
import torch

from oracle import decode, quant, select


def _bf16(x):
    return quant.bf16_to_f32(quant.bf16_bits(np.asarray(x, np.float32)))


def _head(seed, n, D):
    rng = np.random.default_rng(seed)
    sc = rng.lognormal(0, 0.5, D).astype(np.float32)
    sc[rng.choice(D, 2, replace=False)] *= 8
    k = _bf16(rng.standard_normal((n, D)).astype(np.float32) * sc)
    v = _bf16(rng.standard_normal((n, D)).astype(np.float32))
    return k, v


def _sdpa(q, K, V):
    """torch SDPA (fp64) with GQA by repeat_interleave; q [Hq][D], K,V [Hkv][T][D]."""
    Hq = q.shape[0]
    G = Hq // K.shape[0]
    Kt = torch.tensor(K).repeat_interleave(G, 0)
    Vt = torch.tensor(V).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, None, :], Kt, Vt)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("group", [32, 16])
@pytest.mark.parametrize("bits", [2, 4])
def test_decode_matches_torch_sdpa(bits, group):
    n, D, Hkv, G, R = 150, 64, 2, 2, 16
    caches, Ks, Vs = [], [], []
    for j in range(Hkv):
        k, v = _head(j, n, D)
        kept = np.sort(np.random.default_rng(j).choice(n - 8, 70, replace=False))
        kept = np.concatenate([kept, np.arange(n - 8, n)])
        caches.append(quant.build_head_cache(k, v, kept, R, bits, group))
    rng = np.random.default_rng(11)
    q = rng.standard_normal((Hkv * G, D))
    kn = quant.bf16_bits(rng.standard_normal((Hkv, D)).astype(np.float32))
    vn = quant.bf16_bits(rng.standard_normal((Hkv, D)).astype(np.float32))
    out, new = decode.decode_step(caches, q, kn, vn, R, bits)
    for j in range(Hkv):
        K, V = decode.head_keys_values(new[j], bits)
        Ks.append(K)
        Vs.append(V)
    ref = _sdpa(q, np.stack(Ks), np.stack(Vs))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # convex combination of the values attended to
    for h in range(Hkv * G):
        V = Vs[h // G]
        assert np.all(out[h] >= V.min(0) - 1e-12) and np.all(out[h] <= V.max(0) + 1e-12)


def test_dense_special_case_equals_plain_attention():
    # budget >= n - W keeps everything, R >= T quantizes nothing: the step is
    # plain attention over all n+1 bf16 tokens
    n, D, W, Hq, Hkv = 40, 32, 4, 4, 2
    rng = np.random.default_rng(3)
    k = _bf16(rng.standard_normal((1, Hkv, n, D)))
    v = _bf16(rng.standard_normal((1, Hkv, n, D)))
    qw = _bf16(rng.standard_normal((1, Hq, W, D)))
    idx, _ = select.select(qw, k, W, 3, n)           # budget >= n - W
    caches = [quant.build_head_cache(k[0, j], v[0, j], quant.kept_positions(n, W, idx[0, j]),
                                     residual=n, bits=2) for j in range(Hkv)]
    assert all(c["q_len"] == 0 for c in caches)
    q = _bf16(rng.standard_normal((Hq, D)))
    kn = quant.bf16_bits(rng.standard_normal((Hkv, D)))
    vn = quant.bf16_bits(rng.standard_normal((Hkv, D)))
    out, _ = decode.decode_step(caches, q, kn, vn, n, 2)
    Kall = np.concatenate([k[0], quant.bf16_to_f32(kn)[:, None, :]], axis=1).astype(np.float64)
    Vall = np.concatenate([v[0], quant.bf16_to_f32(vn)[:, None, :]], axis=1).astype(np.float64)
    np.testing.assert_allclose(out, _sdpa(q.astype(np.float64), Kall, Vall), rtol=1e-12, atol=1e-14)


def test_blog_masked_hook_semantics():
    # the blog's hook: one softmax over rounded older keys and exact recent keys,
    # output = weights on recent tokens @ exact V + weights on older @ rounded V
    n, D, R, bits = 100, 64, 20, 2
    k, v = _head(5, n, D)
    c = quant.build_head_cache(k, v, np.arange(n), R, bits)
    Q = c["q_len"]
    Kq = np.concatenate([quant.unpack_keys(c["k_codes"], c["k_meta"], bits), k[Q:]])
    Vq = np.concatenate([quant.unpack_values(c["v_codes"], c["v_meta"], bits), v[Q:]])
    q = np.random.default_rng(1).standard_normal(D)
    near = torch.arange(n) >= Q
    qt = torch.tensor(q)
    s = torch.where(near, torch.tensor(k, dtype=torch.float64) @ qt,
                    torch.tensor(Kq, dtype=torch.float64) @ qt) / math.sqrt(D)
    w = torch.softmax(s, -1)
    ref = (w * near) @ torch.tensor(v, dtype=torch.float64) + (w * ~near) @ torch.tensor(Vq, dtype=torch.float64)
    K, V = decode.head_keys_values(c, bits)
    np.testing.assert_allclose(decode.attend(q, K, V), ref.numpy(), rtol=1e-12)


@pytest.mark.parametrize("group", [32, 16])
@pytest.mark.parametrize("T,R,steps", [(72, 16, 70), (44, 128, 130), (300, 128, 40)])
def test_incremental_flush_equals_batch_quantization(T, R, steps, group):
    n, D, bits, g = T, 64, 2, group
    k, v = _head(T, n + steps, D)
    c = quant.build_head_cache(k[:n], v[:n], np.arange(n), R, bits, g)
    flushes = 0
    for s in range(steps):
        before = c["q_len"]
        c = quant.append_and_flush(c, quant.bf16_bits(k[n + s]), quant.bf16_bits(v[n + s]), R, bits)
        flushes += c["q_len"] != before
        assert R <= c["r_len"] < R + g or (c["q_len"] == 0 and c["r_len"] < R + g)
    ref = quant.build_head_cache(k, v, np.arange(n + steps), R, bits, g)
    assert c["q_len"] == ref["q_len"] and c["r_len"] == ref["r_len"]
    for key in ("k_codes", "k_meta", "v_codes", "v_meta", "k_res", "v_res"):
        np.testing.assert_array_equal(c[key], ref[key])
    assert flushes == (ref["q_len"] - quant.build_head_cache(k[:n], v[:n], np.arange(n), R, bits, g)["q_len"]) // g


def test_residual_split_rule():
    k, v = _head(0, 600, 32)
    for T, R in [(72, 16), (276, 128), (44, 128), (544, 128), (32, 0), (160, 128)]:
        c = quant.build_head_cache(k, v, np.arange(T), R, 2)
        assert c["q_len"] % 32 == 0 and c["q_len"] + c["r_len"] == T
        assert c["q_len"] == 32 * (max(T - R, 0) // 32)
    c = quant.build_head_cache(k, v, np.arange(72), 16, 2)
    assert (c["q_len"], c["r_len"]) == (32, 40)


def test_residual_split_rule_group16():
    """MiniKV's group of 16 (Sec. 5.1): Q = 16*floor(max(T-R,0)/16), so the
    residual holds R..R+15 tokens."""
    k, v = _head(0, 600, 32)
    for T, R, want in [(72, 16, (48, 24)), (276, 128, (144, 132)), (44, 128, (0, 44)), (544, 128, (416, 128)),
                       (16, 0, (16, 0)), (175, 128, (32, 143))]:
        c = quant.build_head_cache(k, v, np.arange(T), R, 2, 16)
        assert (c["q_len"], c["r_len"]) == want, (T, R)
        assert c["k_meta"].shape == (want[0] // 16, 32) and c["v_meta"].shape == (want[0], 2)



def test_flush_all_prefill_split_closed_forms():
    """MiniKV Alg. 1 as printed: the prefill quantizes every complete group of
    the kept cache (Q = g*floor(T/g)), so fewer than g tokens stay in bf16."""
    k, v = _head(1, 600, 32)
    for T, g, want in [(72, 32, (64, 8)), (44, 32, (32, 12)), (72, 16, (64, 8)), (31, 32, (0, 31)), (160, 16, (160, 0))]:
        c = quant.build_head_cache(k, v, np.arange(T), 128, 2, g, flush_all=True)
        assert (c["q_len"], c["r_len"]) == want, (T, g)


@pytest.mark.parametrize("group,R", [(32, 64), (16, 48), (16, 16)])
def test_flush_all_incremental_equals_batch_quantization(group, R):
    """Whole-residual flushes: the residual cycles through 0..R-1 tokens, each
    flush quantizes R (a multiple of g) at a group boundary, so the packed
    history always equals the batch quantization of the same token prefix and
    the residual holds the rest."""
    n, D, bits, steps = 100, 64, 2, 150
    k, v = _head(7, n + steps, D)
    c = quant.build_head_cache(k[:n], v[:n], np.arange(n), R, bits, group, flush_all=True)
    flushes = 0
    for s in range(steps):
        before = c["q_len"]
        c = quant.append_and_flush(c, quant.bf16_bits(k[n + s]), quant.bf16_bits(v[n + s]), R, bits)
        if c["q_len"] != before:
            flushes += 1
            assert c["q_len"] - before == R and c["r_len"] == 0
        assert 0 <= c["r_len"] < max(R, (n % group) + 1 + s)
        total = n + s + 1
        assert c["q_len"] + c["r_len"] == total
        kc, km, vc, vm = quant.quantize_tokens(k[:c["q_len"]], v[:c["q_len"]], bits, group)
        for key, ref in (("k_codes", kc), ("k_meta", km), ("v_codes", vc), ("v_meta", vm)):
            np.testing.assert_array_equal(c[key], ref, f"step {s} {key}")
        np.testing.assert_array_equal(c["k_res"], quant.bf16_bits(k[c["q_len"]:total]))
    assert flushes == (steps + n % group) // R


def test_flush_all_decode_matches_torch_sdpa():
    n, D, Hkv, G, R, bits = 90, 64, 2, 2, 32, 4
    caches = [quant.build_head_cache(*_head(20 + j, n, D), np.arange(n), R, bits, 16, flush_all=True)
              for j in range(Hkv)]
    rng = np.random.default_rng(21)
    for s in range(40):
        q = rng.standard_normal((Hkv * G, D))
        kn = quant.bf16_bits(rng.standard_normal((Hkv, D)).astype(np.float32))
        vn = quant.bf16_bits(rng.standard_normal((Hkv, D)).astype(np.float32))
        out, caches = decode.decode_step(caches, q, kn, vn, R, bits)
        Ks, Vs = zip(*(decode.head_keys_values(c, bits) for c in caches))
        np.testing.assert_allclose(out, _sdpa(q, np.stack(Ks), np.stack(Vs)), rtol=1e-12, atol=1e-14)
