"""Oracle: group quantization, bit packing, the kept-cache builder and the
residual flush.  Test infrastructure (see the package docstring).

Cache layout (both sides use it, so "bit-exact packed codes" is well defined):
  k_codes [Q][D*b/32] uint32  word w of token t: channel (32/b)*w+i at bits b*i
  k_meta  [Q/32][D]   uint32  group g (tokens 32g..32g+31), channel c
  v_codes [Q*b/32][D] uint32  word row w, channel c: token (32/b)*w+i at bits b*i
  v_meta  [Q][D/32]   uint32  token t, channel group j (channels 32j..32j+31)
  meta word = fp16 scale bits | (fp16 zero bits << 16)
  k_res, v_res [r][D] uint16  bfloat16 bits, oldest token first
Keys are grouped per channel over 32 tokens and values per token over 32
channels (blog, "Quantization: keep each token in fewer bits": KIVI's grouping;
MiniKV Sec. 4.1).  Codes are packed LSB-first, 16 (2-bit) or 8 (4-bit) per
32-bit word (MiniKV Sec. 4.4, INT2 quantization kernel).
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
    """float32 -> float16 bits, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- one group
def quantize_group(x, bits):
    """Asymmetric min/max quantization of one group of 32 float32 values.

    Blog, "Measured on a real model", ``round_to``: lo/hi per group, step
    (hi-lo)/(2^b-1), codes round((x-lo)/step).  MiniKV Sec. 4.4: zero-point and
    scale are stored as FP16.  Reading fixed for bit-exactness: scale and zero
    are rounded to fp16 first and the codes use the stored values;
    t = (x - zero) * (1/scale) with one fp32 reciprocal per group; codes round
    half to even and clamp to [0, 2^b-1]; a zero (or non-finite) scale gives all
    codes 0.  Every arithmetic step is one IEEE float32 operation.

    Returns (scale_bits uint16, zero_bits uint16, codes uint32[len(x)]).
    """
    x = np.asarray(x, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    lo = x.min()
    hi = x.max()
    s_bits = f16_bits(np.float32(np.float32(hi - lo) / qmax))
    z_bits = f16_bits(lo)
    s = f16_to_f32(s_bits)
    z = f16_to_f32(z_bits)
    if s == 0 or not np.isfinite(s):
        return s_bits, z_bits, np.zeros(x.shape, dtype=np.uint32)
    inv = np.float32(np.float32(1.0) / s)
    t = ((x - z).astype(np.float32) * inv).astype(np.float32)
    codes = np.clip(np.rint(t), 0, qmax).astype(np.uint32)
    return s_bits, z_bits, codes


def meta_word(s_bits, z_bits):
    return np.uint32(int(s_bits)) | (np.uint32(int(z_bits)) << np.uint32(16))


def dequant(codes, s_bits, z_bits):
    """x_hat = zero + code*scale, evaluated in float32 (MiniKV Alg. 1, q^-1)."""
    s = f16_to_f32(s_bits)
    z = f16_to_f32(z_bits)
    return (z + np.asarray(codes, dtype=np.float32) * s).astype(np.float32)


# ---------------------------------------------------------------- packing
def pack_words(codes, bits):
    """Pack a 1-D run of 32/b codes into one uint32, LSB first."""
    per = 32 // bits
    assert len(codes) == per
    w = 0
    for i, c in enumerate(codes):
        w |= int(c) << (bits * i)
    return np.uint32(w)


def quantize_tokens(Kt, Vt, bits):
    """Quantize a whole number of 32-token groups of kept keys/values.

    Kt, Vt: float32 [Q][D] (Q a multiple of 32).  Keys: one group per (32-token
    block, channel); values: one group per (token, 32-channel block).
    Returns k_codes, k_meta, v_codes, v_meta in the layout of the module doc.
    """
    Q, D = Kt.shape
    assert Q % GROUP == 0 and D % GROUP == 0
    per = 32 // bits
    kc = np.zeros((Q, D), dtype=np.uint32)
    vc = np.zeros((Q, D), dtype=np.uint32)
    k_meta = np.zeros((Q // GROUP, D), dtype=np.uint32)
    v_meta = np.zeros((Q, D // GROUP), dtype=np.uint32)
    for g in range(Q // GROUP):
        for c in range(D):
            s, z, codes = quantize_group(Kt[g * GROUP:(g + 1) * GROUP, c], bits)
            k_meta[g, c] = meta_word(s, z)
            kc[g * GROUP:(g + 1) * GROUP, c] = codes
    for t in range(Q):
        for j in range(D // GROUP):
            s, z, codes = quantize_group(Vt[t, j * GROUP:(j + 1) * GROUP], bits)
            v_meta[t, j] = meta_word(s, z)
            vc[t, j * GROUP:(j + 1) * GROUP] = codes
    k_codes = np.zeros((Q, D // per), dtype=np.uint32)
    for t in range(Q):
        for w in range(D // per):
            k_codes[t, w] = pack_words(kc[t, w * per:(w + 1) * per], bits)
    v_codes = np.zeros((Q // per, D), dtype=np.uint32)
    for w in range(Q // per):
        for c in range(D):
            v_codes[w, c] = pack_words(vc[w * per:(w + 1) * per, c], bits)
    return k_codes, k_meta, v_codes, v_meta


def unpack_keys(k_codes, k_meta, bits):
    """Dequantized keys float32 [Q][D] from the packed layout."""
    Q, nw = k_codes.shape
    per = 32 // bits
    D = nw * per
    out = np.zeros((Q, D), dtype=np.float32)
    mask = (1 << bits) - 1
    for t in range(Q):
        for c in range(D):
            code = (int(k_codes[t, c // per]) >> (bits * (c % per))) & mask
            m = int(k_meta[t // GROUP, c])
            out[t, c] = dequant(code, m & 0xFFFF, m >> 16)
    return out


def unpack_values(v_codes, v_meta, bits):
    """Dequantized values float32 [Q][D] from the packed layout."""
    nrow, D = v_codes.shape
    per = 32 // bits
    Q = nrow * per
    out = np.zeros((Q, D), dtype=np.float32)
    mask = (1 << bits) - 1
    for t in range(Q):
        for c in range(D):
            code = (int(v_codes[t // per, c]) >> (bits * (t % per))) & mask
            m = int(v_meta[t, c // GROUP])
            out[t, c] = dequant(code, m & 0xFFFF, m >> 16)
    return out


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


def build_head_cache(k_head, v_head, kept, residual, bits):
    """Prompt compression of one (batch, KV head): gather, quantize, residual.

    MiniKV Alg. 1 prefill (heavy hitters, then Quant); blog "Quantization":
    the most recent tokens stay in full precision until a group fills.  Reading:
    Q = 32*floor(max(T-R,0)/32) oldest kept tokens are quantized, the last T-Q
    (R <= T-Q < R+32 when T >= R) stay as bf16.
    k_head, v_head: float32 [n][D].  Returns a dict.
    """
    T = len(kept)
    Q = GROUP * (max(T - residual, 0) // GROUP)
    Kk = k_head[kept].astype(np.float32)
    Vk = v_head[kept].astype(np.float32)
    kc, km, vc, vm = quantize_tokens(Kk[:Q], Vk[:Q], bits)
    return {
        "q_len": Q, "r_len": T - Q,
        "k_codes": kc, "k_meta": km, "v_codes": vc, "v_meta": vm,
        "k_res": bf16_bits(Kk[Q:]), "v_res": bf16_bits(Vk[Q:]),
    }


def append_and_flush(cache, k_new_bits, v_new_bits, residual, bits):
    """One decode-step cache update (before attention).

    MiniKV Alg. 1 decoding: the new key/value join the fp residual; when it
    reaches its limit it is quantized and concatenated to the packed history.
    Reading: the residual holds R..R+31 tokens; when an append makes it R+32 the
    oldest 32 are quantized (the arithmetic of ``quantize_group``) and appended
    as one group.  k_new_bits/v_new_bits: bf16 bits [D].  Returns a new dict.
    """
    c = dict(cache)
    c["k_res"] = np.concatenate([cache["k_res"], k_new_bits[None, :]], axis=0)
    c["v_res"] = np.concatenate([cache["v_res"], v_new_bits[None, :]], axis=0)
    c["r_len"] = cache["r_len"] + 1
    if c["r_len"] == residual + GROUP:
        Kf = bf16_to_f32(c["k_res"][:GROUP])
        Vf = bf16_to_f32(c["v_res"][:GROUP])
        kc, km, vc, vm = quantize_tokens(Kf, Vf, bits)
        c["k_codes"] = np.concatenate([cache["k_codes"], kc], axis=0)
        c["k_meta"] = np.concatenate([cache["k_meta"], km], axis=0)
        c["v_codes"] = np.concatenate([cache["v_codes"], vc], axis=0)
        c["v_meta"] = np.concatenate([cache["v_meta"], vm], axis=0)
        c["k_res"] = c["k_res"][GROUP:]
        c["v_res"] = c["v_res"][GROUP:]
        c["q_len"] = cache["q_len"] + GROUP
        c["r_len"] -= GROUP
    return c
