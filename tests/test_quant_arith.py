"""Host checks of the float32 identities the GPU quantizer relies on (no GPU).

The quantizer (csrc/quantize.hip, csrc/kvc_internal.h) avoids division
sequences and integer rounding instructions; each shortcut must give exactly
the IEEE float32 result that the oracle's numpy arithmetic gives (MiniKV
Sec. 4.4: fp16 scale and zero-point per group; codes round((x - z) / s)):

* (hi - lo) / qmax as q0 = RN((hi - lo) * c), c = RN(1/qmax), corrected once
  with the exact remainder: RN(q0 + RN(fma(-q0, qmax, d)) * c) as one fma;
* 1/s for an fp16 scale s as one Newton step from any estimate within 2 ulp;
* rint(clamp(t, 0, qmax)) as the low mantissa bits of clamp(t) + 1.5 * 2^23;
* a packed word as a wrapping sum of those bit patterns, less a constant.

Fused multiply-adds are emulated exactly: products of two float32 values are
exact in float64, and the float64 sum's rounding error is recovered by TwoSum,
so a float64 result that lands exactly on a float32 midpoint can be resolved
from the sign of that error.  The division check runs on a dense sample here;
with KVC_EXHAUSTIVE=1 it runs over every finite d >= 0 (about two minutes per
qmax)."""

import os

import numpy as np
import pytest


def _two_sum(a, b):
    s = a + b
    bb = s - a
    return s, (a - (s - bb)) + (b - bb)


def _rn32_exact(s, err):
    """Round the exact value s + err (s = RN64 of it) to float32."""
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    # s exactly halfway between two float32 values: numpy chose the even one,
    # the exact value lies on err's side of s
    tie_up = (s == (r64 + up) / 2) & (err != 0)
    tie_dn = (s == (r64 + dn) / 2) & (err != 0)
    r = np.where(tie_up & (err > 0), up.astype(np.float32), r)
    r = np.where(tie_dn & (err < 0), dn.astype(np.float32), r)
    return r


def _fma32(a, b, c):
    """float32 fma(a, b, c), exactly rounded once."""
    p = a.astype(np.float64) * b.astype(np.float64)  # exact: 24 x 24 bits
    s, err = _two_sum(p, c.astype(np.float64))
    return _rn32_exact(s, err)


def _check_division(d, qmax):
    qm = np.float32(qmax)
    c = np.float32(1.0) / qm
    with np.errstate(over="ignore", invalid="ignore"):
        q0 = (d * c).astype(np.float32)
        r = _fma32(-q0, np.full_like(d, qm), d)
        q1 = _fma32(r, np.full_like(d, c), q0)
        q1 = np.where(np.isfinite(q0), q1, q0)  # d = inf: the kernel keeps q0
        ref = (d / qm).astype(np.float32)
    bad = q1.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), (qmax, d[bad][:5], q1[bad][:5], ref[bad][:5])


def _division_samples(rng):
    blocks = [np.arange(0, 1 << 20, dtype=np.uint32),                      # zero and subnormals
              np.arange(0x3F800000, 0x3F800000 + (1 << 22), dtype=np.uint32),  # [1, 2) in full
              np.arange(0x7F7FFFFF - (1 << 20), 0x7F800001, dtype=np.uint32),   # the top, and +inf
              rng.integers(0, 0x7F800000, size=1 << 22, dtype=np.uint32)]
    return np.concatenate(blocks).view(np.float32)


@pytest.mark.parametrize("qmax", [3, 15])
def test_scale_division_corrected_product(qmax):
    rng = np.random.default_rng(qmax)
    if os.environ.get("KVC_EXHAUSTIVE"):
        step = 1 << 25
        for start in range(0, 0x7F800000, step):
            _check_division(np.arange(start, min(start + step, 0x7F800000), dtype=np.uint32).view(np.float32), qmax)
    else:
        _check_division(_division_samples(rng), qmax)


def test_reciprocal_newton_every_fp16_scale():
    s = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)  # positive finite fp16
    ref = (np.float32(1.0) / s).astype(np.float32)
    for k in range(-2, 3):  # the hardware estimate is within 1 ulp; allow 2
        r0 = ref.copy()
        for _ in range(abs(k)):
            r0 = np.nextafter(r0, np.float32(np.inf if k > 0 else -np.inf))
        e = _fma32(-s, r0, np.ones_like(s))
        r1 = _fma32(e, r0, r0)
        assert np.array_equal(r1.view(np.uint32), ref.view(np.uint32)), k


@pytest.mark.parametrize("bits", [2, 4])
def test_rounding_add_codes_and_word_sums(bits):
    qmax = np.float32(2 ** bits - 1)
    rng = np.random.default_rng(bits)
    t = np.concatenate([rng.uniform(-2.0, float(qmax) + 2.0, 1 << 20).astype(np.float32),
                        (np.arange(-8, 2 * int(qmax) + 8) / np.float32(2)).astype(np.float32),  # ties
                        np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)])
    t = np.concatenate([t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(-np.inf))])
    with np.errstate(invalid="ignore"):
        ref = np.clip(np.rint(t), 0, qmax).astype(np.uint32)
        y = (np.minimum(np.maximum(t, np.float32(0)), qmax) + np.float32(12582912.0)).astype(np.float32)
    yb = y.view(np.uint32)
    assert np.array_equal(yb - np.uint32(0x4B400000), ref)
    per = 32 // bits
    n = (len(t) // per) * per
    codes, ys = ref[:n].reshape(-1, per).astype(np.uint64), yb[:n].reshape(-1, per).astype(np.uint64)
    bias = sum(0x4B400000 << (bits * i) for i in range(per)) & 0xFFFFFFFF
    mask = np.uint64(0xFFFFFFFF)
    word_or, word_sum = np.zeros(len(codes), np.uint64), np.zeros(len(codes), np.uint64)
    for i in range(per):
        word_or |= codes[:, i] << np.uint64(bits * i)
        word_sum = (word_sum + (ys[:, i] << np.uint64(bits * i))) & mask
    assert np.array_equal(word_or, (word_sum - np.uint64(bias)) & mask)
