"""Oracle: per-layer token budgets and cache footprint (host arithmetic only).

Test infrastructure (see the package docstring); exact rational arithmetic so
that the integer budgets have no floating-point tie ambiguity.
"""

from fractions import Fraction
import math


def uniform_budgets(layers, avg):
    """Uniform policy: every layer keeps ``avg`` selected tokens.

    MiniKV, Sec. 4.2 ("Uniform": all layers have the same budget).
    """
    return [int(avg)] * int(layers)


def pyramid_budgets(layers, avg, beta):
    """Arithmetic-pyramid policy with mean exactly ``avg``.

    PyramidKV, Sec. "Proposed Method" (budget allocation): the top layer gets
    total/(beta*m), the rest follow an arithmetic sequence (its closing formula
    is missing from the page).  MiniKV, Sec. 4.2 ("Pyramid"): a linear function
    across layers whose endpoints x/d and 2x - x/d average exactly x; lower
    layers get more.  Reading taken here: top = avg/beta, bottom = 2*avg - top,
    linear in between, layer 0 largest.  Integerization: floor, then +1 to the
    layers with the largest fractional parts (ties to the lower layer), so the
    integer budgets sum to exactly layers*avg.
    """
    L = int(layers)
    if L == 1:
        return [int(avg)]
    b = Fraction(beta)  # exact value of the binary float
    top = Fraction(avg) / b
    bot = 2 * Fraction(avg) - top
    xs = [bot - (bot - top) * Fraction(l, L - 1) for l in range(L)]
    fl = [math.floor(x) for x in xs]
    fr = [x - f for x, f in zip(xs, fl)]
    extra = L * int(avg) - sum(fl)
    order = sorted(range(L), key=lambda l: (-fr[l], l))
    for l in order[:extra]:
        fl[l] += 1
    return fl


def layer_budgets(layers, avg, pyramid, beta, prompt_len, window):
    """Budgets actually applied per layer: policy, then capped at n - W.

    A negative ``avg`` means no eviction: every candidate is kept.  The window
    (PyramidKV's last alpha "instruction tokens") is kept on top of the budget.
    """
    cand = prompt_len - window
    if avg < 0:
        return [cand] * layers
    ks = pyramid_budgets(layers, avg, beta) if pyramid else uniform_budgets(layers, avg)
    return [min(k, cand) for k in ks]


def weighted_budgets(weights, avg):
    """Budgets proportional to positive per-layer weights, mean ``avg``.

    MiniKV, Sec. 4.2, the variance policies: Var-prop gives a layer a share of
    the cache proportional to the variance of its cumulated attention, Var-inv
    a share inversely proportional to it (so the weight is the variance or its
    reciprocal).  Readings: the shares are x_l = L*avg*w_l / sum(w), so that the
    mean is avg; integerization as for the pyramid (floor, then +1 to the layers
    with the largest fractional parts, ties to the lower layer), with the
    shares computed in IEEE double in this order: S = w_0 + w_1 + ... (left to
    right), x_l = (L*avg * w_l) / S.  The +1s go to at most L layers and at
    least none, so the sum is L*avg whenever the rounding of S leaves the
    floors' deficit in [0, L].
    """
    w = [float(x) for x in weights]
    L = len(w)
    S = 0.0
    for x in w:
        S = S + x
    tot = float(L * int(avg))
    xs = [(tot * x) / S for x in w]
    fl = [math.floor(x) for x in xs]
    fr = [x - f for x, f in zip(xs, fl)]
    extra = min(max(L * int(avg) - sum(fl), 0), L)
    order = sorted(range(L), key=lambda l: (-fr[l], l))
    for l in order[:extra]:
        fl[l] += 1
    return fl


def weighted_layer_budgets(weights, avg, prompt_len, window):
    """Weighted budgets capped at the n - W candidates (as layer_budgets)."""
    cand = prompt_len - window
    return [min(k, cand) for k in weighted_budgets(weights, avg)]


def bits_per_element(bits, group, meta_bits):
    """Storage bits per cached number.

    Blog, "The budget": a 16-bit scale and zero-point per 32 numbers adds one bit
    per number.  MiniKV, "KV Cache compression ratio analysis": group 16 at 2 bits
    costs 16*2 bits + 2*2 bytes = 8 bytes per 16 numbers.  16 bits = unquantized.
    """
    if bits == 16:
        return 16.0
    return bits + 2.0 * meta_bits / group


def kept_tokens(layers, avg, pyramid, beta, prompt_len, window):
    """Kept prompt tokens per layer per KV head: selected + window (or all n)."""
    if avg < 0:
        return [prompt_len] * layers
    return [k + window for k in layer_budgets(layers, avg, pyramid, beta, prompt_len, window)]


def footprint(layers, kv_heads, head_dim, prompt_len, window, gen_len, avg, pyramid,
              beta, bits, group, meta_bits, residual):
    """Cache footprint for one sequence.

    bytes_per_prompt_token: the blog's formula 2*L*H*D*bits/8 scaled by the
        kept fraction of the prompt (blog, "The budget").
    bytes_total: 2*H*D*bits/8 summed over layers of (kept + generated) tokens
        (MiniKV, "KV Cache compression ratio analysis").
    bytes_layout: exact bytes of the packed layout right after prompt
        compression: codes + fp16 scale/zero + bf16 residual, per layer and head,
        with Q = g*floor(max(T-R,0)/g) quantized and T-Q residual tokens.
    """
    bpe = bits_per_element(bits, group, meta_bits)
    T = kept_tokens(layers, avg, pyramid, beta, prompt_len, window)
    frac = sum(T) / (layers * prompt_len)
    per_tok = 2.0 * layers * kv_heads * head_dim * bpe / 8.0
    total = 2.0 * kv_heads * head_dim * bpe / 8.0 * sum(t + gen_len for t in T)
    lay = 0
    for t in T:
        if bits == 16:
            lay += 2 * t * head_dim * 2
            continue
        q = group * (max(t - residual, 0) // group)
        codes = 2 * q * head_dim * bits // 8
        pair = 2 * meta_bits // 8  # one scale + one zero-point
        meta = (q // group) * head_dim * pair + q * (head_dim // group) * pair
        res = 2 * (t - q) * head_dim * 2
        lay += codes + meta + res
    return {
        "bits_per_element": bpe,
        "bytes_per_prompt_token": per_tok * frac,
        "bytes_total": total,
        "bytes_layout": float(lay * kv_heads),
    }
