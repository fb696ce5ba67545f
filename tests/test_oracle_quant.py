"""Pins of the oracle's group quantizer and packer: the error bound, exact
nearest-level brute force, integer groups, the blog's rounding semantics and an
independent unpack of the bit layout."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant


def _groups(seed, count, kind):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((count, 32)).astype(np.float32)
    x *= rng.lognormal(0, 1.5, size=(count, 1)).astype(np.float32)
    if kind == "bf16":
        x = quant.bf16_to_f32(quant.bf16_bits(x))
    return x


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_dequant_error_bound(bits, kind):
    for x in _groups(bits * 10 + len(kind), 400, kind):
        s_b, z_b, codes = quant.quantize_group(x, bits)
        s = float(quant.f16_to_f32(s_b))
        z = float(quant.f16_to_f32(z_b))
        xh = quant.dequant(codes, s_b, z_b).astype(np.float64)
        lo = float(x.min())
        bound = s * (0.5 + 2 ** -16) + abs(z - lo) + 2 ** -22 * np.maximum(np.abs(x), abs(z))
        assert np.all(np.abs(x - xh) <= bound + 1e-30)
        if kind == "bf16":
            assert z == lo   # bf16 values in fp16's normal range are exact in fp16


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_exact_nearest_levels(bits):
    qmax = 2 ** bits - 1
    for x in _groups(100 + bits, 300, "bf16"):
        s_b, z_b, codes = quant.quantize_group(x, bits)
        s = Fraction(float(quant.f16_to_f32(s_b)))
        z = Fraction(float(quant.f16_to_f32(z_b)))
        for xi, ci in zip(x, codes):
            t = (Fraction(float(xi)) - z) / s
            fl = t.numerator // t.denominator
            frac = t - fl
            if abs(frac - Fraction(1, 2)) <= Fraction(1, 2 ** 18):
                ok = {min(max(fl, 0), qmax), min(max(fl + 1, 0), qmax)}
            else:
                ok = {min(max(fl + (1 if frac > Fraction(1, 2) else 0), 0), qmax)}
            assert int(ci) in ok


def test_integer_groups_exact():
    s_b, z_b, c = quant.quantize_group(np.array([0, 1, 2, 3] * 8, np.float32), 2)
    assert int(s_b) == 0x3C00 and int(z_b) == 0 and list(c) == [0, 1, 2, 3] * 8
    s_b, z_b, c = quant.quantize_group(np.arange(32, dtype=np.float32) % 16 - 8, 4)
    assert float(quant.f16_to_f32(s_b)) == 1.0 and float(quant.f16_to_f32(z_b)) == -8.0
    assert list(c) == list(range(16)) * 2
    # constant group: zero scale, all codes 0, exact reconstruction
    s_b, z_b, c = quant.quantize_group(np.full(32, -0.75, np.float32), 2)
    assert int(s_b) == 0 and not c.any()
    assert np.all(quant.dequant(c, s_b, z_b) == -0.75)
    # halfway values round to even levels
    s_b, z_b, c = quant.quantize_group(np.array([0, 3, 0.5, 1.5, 2.5] + [0] * 27, np.float32), 2)
    assert list(c[:5]) == [0, 3, 0, 2, 2]


def _blog_rounding(x, bits, per, group):
    """The blog's rounding semantics (round_to), restated: asymmetric min/max per
    group; per token = groups of channels, per channel = groups of tokens."""
    t, c = x.shape
    if per == "token":
        g = x.view(t, c // group, group)
        lo = g.min(dim=-1, keepdim=True).values
        hi = g.max(dim=-1, keepdim=True).values
    else:
        g = x.view(t // group, group, c)
        lo = g.min(dim=1, keepdim=True).values
        hi = g.max(dim=1, keepdim=True).values
    s = torch.clamp(hi - lo, min=1e-8) / (2 ** bits - 1)
    return (torch.round((g - lo) / s) * s + lo).view(t, c)


@pytest.mark.parametrize("bits", [2, 4])
def test_matches_blog_round_to_where_scales_are_fp16_exact(bits):
    rng = np.random.default_rng(5)
    T, D = 64, 64
    qmax = 2 ** bits - 1
    # build groups whose min and step are exact in fp16 and whose step is a power
    # of two, so that dividing and multiplying by the reciprocal agree exactly
    K = np.zeros((T, D), np.float32)
    for g in range(T // 32):
        for c in range(D):
            lo = rng.integers(-64, 64) / 8
            step = 2.0 ** rng.integers(-3, 2)
            vals = lo + rng.integers(0, qmax * 8 + 1, 32) * step / 8
            vals[0], vals[1] = lo, lo + qmax * step
            K[32 * g:32 * g + 32, c] = vals
    V = np.ascontiguousarray(K.T[:T, :D]) if T == D else K.copy()
    kc, km, vc, vm = quant.quantize_tokens(K, V, bits)
    Kh = quant.unpack_keys(kc, km, bits)
    ref = _blog_rounding(torch.tensor(K), bits, "channel", 32).numpy()
    np.testing.assert_array_equal(Kh, ref)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_layout_independent_unpack(bits):
    rng = np.random.default_rng(9)
    Q, D = 64, 64
    K = rng.standard_normal((Q, D)).astype(np.float32)
    V = rng.standard_normal((Q, D)).astype(np.float32)
    kc, km, vc, vm = quant.quantize_tokens(K, V, bits)
    per, mask = 32 // bits, (1 << bits) - 1
    assert kc.shape == (Q, D // per) and vc.shape == (Q // per, D)
    assert km.shape == (Q // 32, D) and vm.shape == (Q, D // 32)
    shifts = (np.arange(per, dtype=np.uint32) * bits)
    # keys: word w of token t holds channels per*w + i
    kcodes = ((kc[:, :, None] >> shifts) & mask).reshape(Q, D)
    # values: word row w of channel c holds tokens per*w + i
    vcodes = ((vc[:, None, :] >> shifts[None, :, None]) & mask).reshape(Q, D)
    for g in range(Q // 32):
        for c in range(D):
            s_b, z_b, codes = quant.quantize_group(K[32 * g:32 * g + 32, c], bits)
            assert np.array_equal(kcodes[32 * g:32 * g + 32, c], codes)
            assert int(km[g, c]) == int(s_b) | (int(z_b) << 16)
    for t in range(Q):
        for j in range(D // 32):
            s_b, z_b, codes = quant.quantize_group(V[t, 32 * j:32 * j + 32], bits)
            assert np.array_equal(vcodes[t, 32 * j:32 * j + 32], codes)
            assert int(vm[t, j]) == int(s_b) | (int(z_b) << 16)


def test_bit_order_worked_example():
    # codes 1,2,3,0,... LSB first -> 1 | 2<<2 | 3<<4 = 57
    assert int(quant.pack_words([1, 2, 3] + [0] * 13, 2)) == 57
    assert int(quant.pack_words([15, 1] + [0] * 6, 4)) == 0x1F


def test_bf16_rounding():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -2.5], np.float32)
    got = quant.bf16_to_f32(quant.bf16_bits(x))
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("bits", [2, 4])
def test_group16_layout_through_packing(bits):
    """Keys grouped per channel over 16 tokens and values per token over 16
    channels (MiniKV's group size), read back through the packed layout: every
    element is within half a step of its own 16-group's scale (plus the fp16
    zero's rounding).  Blocks of 16 tokens and of 16 channels sit at offsets 0
    and 100 alternately, so metadata indexed by 32-wide groups (or by the wrong
    axis) would miss the bound by two orders of magnitude."""
    rng = np.random.default_rng(5 + bits)
    Q, D, g = 64, 64, 16
    K = rng.standard_normal((Q, D)).astype(np.float32) + 100.0 * ((np.arange(Q) // g) % 2)[:, None]
    V = rng.standard_normal((Q, D)).astype(np.float32) + 100.0 * ((np.arange(D) // g) % 2)[None, :]
    kc, km, vc, vm = quant.quantize_tokens(K, V, bits, g)
    assert km.shape == (Q // g, D) and vm.shape == (Q, D // g)
    Kh = quant.unpack_keys(kc, km, bits, g)
    Vh = quant.unpack_values(vc, vm, bits, g)
    qmax = 2 ** bits - 1
    for t in range(Q):
        for c in range(D):
            kb = K[g * (t // g):g * (t // g) + g, c]
            vb = V[t, g * (c // g):g * (c // g) + g]
            for x, xh, blk in ((K[t, c], Kh[t, c], kb), (V[t, c], Vh[t, c], vb)):
                lo, hi = float(blk.min()), float(blk.max())
                s = float(quant.f16_to_f32(quant.f16_bits((hi - lo) / qmax)))
                z = float(quant.f16_to_f32(quant.f16_bits(lo)))
                assert abs(float(x) - float(xh)) <= s * (0.5 + 2 ** -16) + abs(z - lo) + 1e-4 * max(abs(x), 1.0)


def test_group16_integer_groups_exact():
    """Integer-valued 16-groups quantize exactly (scale 1, zero the minimum)."""
    K = np.tile(np.array([0, 1, 2, 3] * 4, np.float32)[:, None], (2, 32)) + np.repeat([0.0, 8.0], 16)[:, None]
    V = np.tile(np.array([5, 6, 7, 8] * 4, np.float32)[None, :], (32, 2))
    kc, km, vc, vm = quant.quantize_tokens(K.astype(np.float32), V.astype(np.float32), 2, 16)
    np.testing.assert_array_equal(quant.unpack_keys(kc, km, 2, 16), K)
    np.testing.assert_array_equal(quant.unpack_values(vc, vm, 2, 16), V)
    assert set((km & 0xFFFF).ravel().tolist()) == {0x3C00} and set(((km >> 16) & 0xFFFF).ravel().tolist()) == {0, 0x4800}
    assert set((vm & 0xFFFF).ravel().tolist()) == {0x3C00} and set((vm >> 16).ravel().tolist()) == {0x4500}

