"""Oracle: group quantization, bit packing, the kept-cache builder and the
residual flush.  Test infrastructure (see the package docstring).

Cache layout (both sides use it, so "bit-exact packed codes" is well defined),
for a group size g (32 by default; MiniKV's own setting is 16):
  k_codes [Q][D*b/32] uint32  word w of token t: channel (32/b)*w+i at bits b*i
  k_meta  [Q/g][D]    uint32  group q (tokens gq..gq+g-1), channel c
  v_codes [Q*b/32][D] uint32  word row w, channel c: token (32/b)*w+i at bits b*i
  v_meta  [Q][D/g]    uint32  token t, channel group j (channels gj..gj+g-1)
  meta word = fp16 scale bits | (fp16 zero bits << 16)
  k_res, v_res [r][D] uint16  bfloat16 bits, oldest token first
Keys are grouped per channel over g tokens and values per token over g
channels (blog, "Quantization: keep each token in fewer bits": KIVI's grouping;
MiniKV Sec. 4.1, and Sec. 5.1 for its group size 16).  Codes are packed
LSB-first, 16 (2-bit) or 8 (4-bit) per 32-bit word (MiniKV Sec. 4.4, INT2
quantization kernel); the packing does not depend on g.
"""

import numpy as np

GROUP = 32


# ---------------------------------------------------------------- number formats
def bf16_bits(x):
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits):
    """bfloat16 bits -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_bits(x):
    """float32 -> float16 bits, round to nearest even (numpy's cast; magnitudes
    past the fp16 range become infinities, as IEEE rounding says)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- groups
def quantize_groups(X, bits):
    """Asymmetric min/max quantization of groups of float32 values.

    X: float32 [..., g], one group per row of the last axis (g = 32 or 16).
    Blog, "Measured on a real model", ``round_to``: lo/hi per group, step
    (hi-lo)/(2^b-1), codes round((x-lo)/step).  MiniKV Sec. 4.4: zero-point and
    scale are stored as FP16.  Reading fixed for bit-exactness: scale and zero
    are rounded to fp16 first and the codes use the stored values;
    t = (x - zero) * (1/scale) with one fp32 reciprocal per group; codes round
    half to even and clamp to [0, 2^b-1]; a zero (or non-finite) scale gives all
    codes 0.  Every arithmetic step is one IEEE float32 operation per element
    (numpy float32 array arithmetic), so rows are independent of each other.

    Returns (scale_bits uint16 [...], zero_bits uint16 [...], codes uint32 [..., g]).
    """
    X = np.asarray(X, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    lo = X.min(axis=-1)
    hi = X.max(axis=-1)
    s_bits = f16_bits((hi - lo).astype(np.float32) / qmax)
    z_bits = f16_bits(lo)
    s = f16_to_f32(s_bits)
    z = f16_to_f32(z_bits)
    ok = (s != 0) & np.isfinite(s)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        inv = (np.float32(1.0) / np.where(ok, s, np.float32(1.0))).astype(np.float32)
        t = ((X - z[..., None]).astype(np.float32) * inv[..., None]).astype(np.float32)
        codes = np.clip(np.rint(t), 0, qmax).astype(np.uint32)
    codes[~ok] = 0
    return s_bits, z_bits, codes


def quantize_group(x, bits):
    """One group of values (``quantize_groups`` on a single row)."""
    s_bits, z_bits, codes = quantize_groups(np.asarray(x, dtype=np.float32)[None], bits)
    return s_bits[0], z_bits[0], codes[0]


def meta_word(s_bits, z_bits):
    """Metadata word(s): fp16 scale bits | fp16 zero bits << 16."""
    return np.asarray(s_bits).astype(np.uint32) | (np.asarray(z_bits).astype(np.uint32) << np.uint32(16))


def dequant(codes, s_bits, z_bits):
    """x_hat = zero + code*scale, evaluated in float32 (MiniKV Alg. 1, q^-1)."""
    s = f16_to_f32(s_bits)
    z = f16_to_f32(z_bits)
    return (z + np.asarray(codes, dtype=np.float32) * s).astype(np.float32)


# ---------------------------------------------------------------- packing
def pack_words(codes, bits):
    """Pack runs of 32/b codes into uint32 words, LSB first.

    codes: [..., 32/b] -> uint32 [...]; code i of a run goes to bits b*i.
    """
    codes = np.asarray(codes, dtype=np.uint64)
    per = 32 // bits
    assert codes.shape[-1] == per
    shifts = (bits * np.arange(per)).astype(np.uint64)
    return np.bitwise_or.reduce(codes << shifts, axis=-1).astype(np.uint32)


def unpack_words(words, bits):
    """Inverse of ``pack_words``: uint32 [...] -> codes uint32 [..., 32/b]."""
    per = 32 // bits
    shifts = (bits * np.arange(per)).astype(np.uint32)
    return (np.asarray(words, dtype=np.uint32)[..., None] >> shifts) & np.uint32((1 << bits) - 1)


def quantize_tokens(Kt, Vt, bits, group=GROUP):
    """Quantize a whole number of g-token groups of kept keys/values.

    Kt, Vt: float32 [Q][D] (Q a multiple of g = group).  Keys: one group per
    (g-token block, channel); values: one group per (token, g-channel block).
    Returns k_codes, k_meta, v_codes, v_meta in the layout of the module doc.
    """
    Q, D = Kt.shape
    g = group
    per = 32 // bits
    assert Q % g == 0 and D % g == 0 and Q % per == 0
    # keys: group (q, c) = Kt[gq:gq+g, c]
    kg = np.ascontiguousarray(Kt.reshape(Q // g, g, D).transpose(0, 2, 1))  # [Q/g][D][g]
    ks, kz, kcodes = quantize_groups(kg, bits)
    k_meta = meta_word(ks, kz)                                        # [Q/g][D]
    kc = kcodes.transpose(0, 2, 1).reshape(Q, D)                      # code of (token, channel)
    # values: group (t, j) = Vt[t, gj:gj+g]
    vs, vz, vcodes = quantize_groups(Vt.reshape(Q, D // g, g), bits)
    v_meta = meta_word(vs, vz)                                        # [Q][D/g]
    vc = vcodes.reshape(Q, D)
    k_codes = pack_words(kc.reshape(Q, D // per, per), bits)          # channels of a token
    v_codes = pack_words(vc.reshape(Q // per, per, D).transpose(0, 2, 1), bits)  # tokens of a channel
    return k_codes, k_meta, v_codes, v_meta


def unpack_keys(k_codes, k_meta, bits, group=GROUP):
    """Dequantized keys float32 [Q][D] from the packed layout."""
    Q, nw = k_codes.shape
    codes = unpack_words(k_codes, bits).reshape(Q, nw * (32 // bits))  # [Q][D]
    m = np.repeat(np.asarray(k_meta, dtype=np.uint32), group, axis=0)  # meta of (t // g, c)
    return dequant(codes, (m & 0xFFFF).astype(np.uint16), (m >> 16).astype(np.uint16))


def unpack_values(v_codes, v_meta, bits, group=GROUP):
    """Dequantized values float32 [Q][D] from the packed layout."""
    nrow, D = v_codes.shape
    codes = unpack_words(v_codes, bits).transpose(0, 2, 1).reshape(nrow * (32 // bits), D)  # [Q][D]
    m = np.repeat(np.asarray(v_meta, dtype=np.uint32), group, axis=1)      # meta of (t, c // g)
    return dequant(codes, (m & 0xFFFF).astype(np.uint16), (m >> 16).astype(np.uint16))


# ---------------------------------------------------------------- cache builder
def as_f32(x, dtype):
    """Model-dtype tensor as float32 values: fp32 as is, bf16 given as bits."""
    if dtype == "bf16":
        return bf16_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def kept_positions(n, W, idx_row):
    """Kept prompt positions: selected ascending, then the window [n-W, n)."""
    if idx_row is None:
        return np.arange(n)
    return np.concatenate([np.asarray(idx_row, dtype=np.int64), np.arange(n - W, n)])


def build_head_cache(k_head, v_head, kept, residual, bits, group=GROUP, flush_all=False):
    """Prompt compression of one (batch, KV head): gather, quantize, residual.

    MiniKV Alg. 1 prefill (heavy hitters, then Quant); blog "Quantization":
    the most recent tokens stay in full precision until a group fills.  Reading:
    Q = g*floor(max(T-R,0)/g) oldest kept tokens are quantized (g = group), the
    last T-Q (R <= T-Q < R+g when T >= R) stay as bf16.  With flush_all (MiniKV
    Alg. 1 as printed: the prefill quantizes the kept cache, the residual only
    collects decoded tokens) Q = g*floor(T/g), so fewer than g tokens remain.
    k_head, v_head: float32 [n][D].  Returns a dict (its "group" is g).
    """
    T = len(kept)
    Q = group * (T // group) if flush_all else group * (max(T - residual, 0) // group)
    Kk = k_head[kept].astype(np.float32)
    Vk = v_head[kept].astype(np.float32)
    kc, km, vc, vm = quantize_tokens(Kk[:Q], Vk[:Q], bits, group)
    return {
        "group": group, "flush_all": flush_all, "q_len": Q, "r_len": T - Q,
        "k_codes": kc, "k_meta": km, "v_codes": vc, "v_meta": vm,
        "k_res": bf16_bits(Kk[Q:]), "v_res": bf16_bits(Vk[Q:]),
    }


def append_and_flush(cache, k_new_bits, v_new_bits, residual, bits):
    """One decode-step cache update (before attention).

    MiniKV Alg. 1 decoding: the new key/value join the fp residual; when it
    reaches its limit it is quantized and concatenated to the packed history.
    Reading: the residual holds R..R+g-1 tokens (g = the cache's group); when an
    append makes it R+g the oldest g are quantized (the arithmetic of
    ``quantize_group``) and appended as one group.  With the cache's flush_all
    (MiniKV Alg. 1 as printed) the residual is instead quantized whole, in
    groups of g, when it reaches R tokens.  k_new_bits/v_new_bits: bf16 bits
    [D].  Returns a new dict.
    """
    g = cache.get("group", GROUP)
    c = dict(cache)
    if cache.get("flush_all", False):
        # MiniKV Alg. 1 decoding: the residual is quantized whole once it holds
        # n_r = R tokens (R a multiple of g), in groups of g, oldest first
        c["k_res"] = np.concatenate([cache["k_res"], k_new_bits[None, :]], axis=0)
        c["v_res"] = np.concatenate([cache["v_res"], v_new_bits[None, :]], axis=0)
        c["r_len"] = cache["r_len"] + 1
        if c["r_len"] == residual:
            kc, km, vc, vm = quantize_tokens(bf16_to_f32(c["k_res"]), bf16_to_f32(c["v_res"]), bits, g)
            c["k_codes"] = np.concatenate([cache["k_codes"], kc], axis=0)
            c["k_meta"] = np.concatenate([cache["k_meta"], km], axis=0)
            c["v_codes"] = np.concatenate([cache["v_codes"], vc], axis=0)
            c["v_meta"] = np.concatenate([cache["v_meta"], vm], axis=0)
            c["k_res"] = c["k_res"][:0]
            c["v_res"] = c["v_res"][:0]
            c["q_len"] = cache["q_len"] + residual
            c["r_len"] = 0
        return c
    c["k_res"] = np.concatenate([cache["k_res"], k_new_bits[None, :]], axis=0)
    c["v_res"] = np.concatenate([cache["v_res"], v_new_bits[None, :]], axis=0)
    c["r_len"] = cache["r_len"] + 1
    if c["r_len"] == residual + g:
        Kf = bf16_to_f32(c["k_res"][:g])
        Vf = bf16_to_f32(c["v_res"][:g])
        kc, km, vc, vm = quantize_tokens(Kf, Vf, bits, g)
        c["k_codes"] = np.concatenate([cache["k_codes"], kc], axis=0)
        c["k_meta"] = np.concatenate([cache["k_meta"], km], axis=0)
        c["v_codes"] = np.concatenate([cache["v_codes"], vc], axis=0)
        c["v_meta"] = np.concatenate([cache["v_meta"], vm], axis=0)
        c["k_res"] = c["k_res"][g:]
        c["v_res"] = c["v_res"][g:]
        c["q_len"] = cache["q_len"] + g
        c["r_len"] -= g
    return c
