"""Pins of the oracle's budget and footprint arithmetic against numbers the
pages print and against the invariants of the pyramid policy."""

import json
import math
import os

import numpy as np
import pytest

from oracle import budget

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _blog_row(shape, heads, bits, frac):
    n = shape["context"]
    avg = -1 if frac == 1.0 else int(frac * n)
    return budget.footprint(layers=shape["layers"], kv_heads=heads, head_dim=shape["head_dim"],
                            prompt_len=n, window=0, gen_len=0, avg=avg, pyramid=False, beta=1.0,
                            bits=bits, group=32, meta_bits=16, residual=0)


def test_blog_budget_table_exact_digits():
    g = _load("blog_budget_table.json")
    shape = g["shape"]
    base = _blog_row(shape, shape["heads"], 16, 1.0)["bytes_per_prompt_token"]
    for heads, bits, frac, b_txt, gib_txt, pct_txt in g["rows"]:
        fp = _blog_row(shape, heads, bits, frac)
        b = fp["bytes_per_prompt_token"]
        assert f"{b:,.0f}" == b_txt
        assert f"{b * shape['context'] / 2**30:.2f}" == gib_txt
        assert f"{b / base:.1%}" == pct_txt


def test_blog_one_bit_overhead_and_800kib():
    # 16-bit scale + 16-bit zero per 32 numbers = +1 bit per number
    assert budget.bits_per_element(2, 32, 16) == 3.0
    assert budget.bits_per_element(4, 32, 16) == 5.0
    fp = _blog_row({"layers": 40, "heads": 40, "head_dim": 128, "context": 32768}, 40, 16, 1.0)
    assert fp["bytes_per_prompt_token"] == 800 * 1024


def test_minikv_worked_example():
    g = _load("minikv_kv_size.json")
    m = g["model"]
    common = dict(layers=m["layers"], kv_heads=m["kv_heads"], head_dim=m["head_dim"],
                  prompt_len=m["prompt"], pyramid=False, beta=1.0, residual=0)
    full = budget.footprint(window=0, gen_len=m["gen"], avg=-1, bits=16, group=16, meta_bits=16, **common)
    # 50% budget: 25% heavy hitters + 25% recent window, 2-bit group 16 (8 B per 16 numbers)
    mini = budget.footprint(window=m["prompt"] // 4, gen_len=m["gen"], avg=m["prompt"] // 4,
                            bits=2, group=16, meta_bits=16, **common)
    # H2O at a 15% budget: fp16, fixed cache size (no generated-token growth)
    h2o = budget.footprint(window=0, gen_len=0, avg=int(0.15 * m["prompt"]), bits=16, group=16,
                           meta_bits=16, **common)
    assert budget.bits_per_element(2, 16, 16) == 4.0  # 8 bytes per 16 numbers
    p = g["printed"]

    def trunc(x, d):  # the page truncates (0.3355 GB is printed as 0.33)
        return f"{math.floor(x * 10**d) / 10**d:.{d}f}"

    assert trunc(full["bytes_total"] / 1e9, 1) == p["full_GB"]
    assert trunc(mini["bytes_total"] / 1e9, 2) == p["minikv_GB"]
    assert trunc(h2o["bytes_total"] / 1e9, 2) == p["h2o_15pct_GB"]
    assert f"{100 * (1 - mini['bytes_total'] / full['bytes_total']):.0f}" == p["compression_pct"]
    # the closed forms of the analysis: full = 2*(H*d)*(lp+lg)*2 B, MiniKV = (H*d)*(a)*lp + (H*d)*lg B
    Hd = m["layers"] * m["kv_heads"] * m["head_dim"]
    assert full["bytes_total"] == 2 * Hd * (m["prompt"] + m["gen"]) * 2
    assert mini["bytes_total"] == Hd * 0.5 * m["prompt"] + Hd * m["gen"]


def test_cskv_and_pyramidkv_claims():
    g = _load("footprint_claims.json")
    c = g["cskv"]
    m = c["model"]
    per_tok = 2 * m["layers"] * m["kv_heads"] * m["head_dim"] * m["bytes"]
    fp = budget.footprint(layers=m["layers"], kv_heads=m["kv_heads"], head_dim=m["head_dim"],
                          prompt_len=c["tokens"], window=0, gen_len=0, avg=-1, pyramid=False,
                          beta=1.0, bits=16, group=32, meta_bits=16, residual=0)
    assert fp["bytes_per_prompt_token"] == per_tok
    total = fp["bytes_total"]
    assert abs(total / 1e9 - c["approx_GB"]) / c["approx_GB"] < 0.1
    assert total / ((c["card_GB"] - c["weights_GB"]) * 1e9) > c["min_ratio"]
    p = g["pyramidkv"]
    fp100k = budget.footprint(layers=32, kv_heads=32, head_dim=128, prompt_len=p["tokens_100k"],
                              window=0, gen_len=0, avg=-1, pyramid=False, beta=1.0, bits=16,
                              group=32, meta_bits=16, residual=0)
    assert fp100k["bytes_total"] > p["over_GB"] * 1e9
    fp2k = budget.footprint(layers=32, kv_heads=32, head_dim=128, prompt_len=p["tokens_2k"],
                            window=0, gen_len=0, avg=-1, pyramid=False, beta=1.0, bits=16,
                            group=32, meta_bits=16, residual=0)
    assert fp2k["bytes_total"] == 2 ** 30


@pytest.mark.parametrize("L,avg,beta", [(32, 128, 10.5), (32, 2048, 10.5), (40, 77, 20.0),
                                        (7, 5, 3.0), (2, 10, 1.0), (33, 1000, 7.25)])
def test_pyramid_invariants(L, avg, beta):
    ks = budget.pyramid_budgets(L, avg, beta)
    assert len(ks) == L
    assert sum(ks) == L * avg                       # mean exactly avg (MiniKV Sec. 4.2)
    assert all(a >= b for a, b in zip(ks, ks[1:]))  # lower layers get more
    top, bot = avg / beta, 2 * avg - avg / beta
    assert abs(ks[-1] - top) < 1 and abs(ks[0] - bot) < 1
    # consecutive steps of an arithmetic sequence differ by at most one after rounding
    steps = [a - b for a, b in zip(ks, ks[1:])]
    assert max(steps) - min(steps) <= 1


def test_pyramid_endpoints_of_the_pages():
    # PyramidKV: top layer k^{m-1} = k_total/(beta*m) = avg/beta
    ks = budget.pyramid_budgets(32, 128, 10.5)
    assert ks[-1] == round(128 / 10.5)
    # MiniKV pyramid: endpoints x/d and 2x - x/d with depth d; mean x
    d = 7
    ks = budget.pyramid_budgets(32, 700, d)
    assert ks[-1] == 100 and ks[0] == 1300 and sum(ks) == 32 * 700
    # the last layer is about 1/20 of the first at beta = 10.5
    ks = budget.pyramid_budgets(32, 2048, 10.5)
    assert abs(ks[-1] / ks[0] - 1 / 20) < 0.001


def test_pyramid_single_layer_is_uniform_and_cap():
    assert budget.pyramid_budgets(1, 77, 20.0) == [77]
    ks = budget.layer_budgets(4, 100, True, 10.5, prompt_len=120, window=8)
    assert max(ks) <= 112
    assert budget.layer_budgets(3, -1, False, 1.0, prompt_len=50, window=5) == [45, 45, 45]


def test_layout_bytes_equal_blog_formula_without_eviction():
    # R = 0, no eviction, n % 32 == 0: the exact layout is the blog formula
    for bits in (2, 4):
        fp = budget.footprint(layers=3, kv_heads=5, head_dim=64, prompt_len=4096, window=1,
                              gen_len=0, avg=-1, pyramid=False, beta=1.0, bits=bits, group=32,
                              meta_bits=16, residual=0)
        assert fp["bytes_layout"] == fp["bytes_per_prompt_token"] * 4096


# ---- weighted budgets (MiniKV Sec. 4.2, Var-prop / Var-inv)

@pytest.mark.parametrize("L,avg", [(1, 7), (5, 128), (32, 512), (40, 3)])
def test_weighted_equal_weights_is_uniform(L, avg):
    assert budget.weighted_budgets([2.5] * L, avg) == [avg] * L


def test_weighted_closed_forms_by_hand():
    # shares 5 and 15 exactly
    assert budget.weighted_budgets([1.0, 3.0], 10) == [5, 15]
    # shares 2/3 and 4/3: floors 0, 1; one +1 to the larger fraction (layer 0)
    assert budget.weighted_budgets([1.0, 2.0], 1) == [1, 1]
    # shares 0.625 x4 and 2.5: floors 0,0,0,0,2; three +1s among four tied
    # fractions go to the lowest layers
    assert budget.weighted_budgets([1.0, 1.0, 1.0, 1.0, 4.0], 1) == [1, 1, 1, 0, 2]
    # Var-inv of variances 1, 2, 4: weights 1, 1/2, 1/4 -> shares 3*7*(4/7, 2/7, 1/7) = 12, 6, 3
    assert budget.weighted_budgets([1.0, 0.5, 0.25], 7) == [12, 6, 3]


@pytest.mark.parametrize("seed", range(6))
def test_weighted_invariants(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(2, 48))
    avg = int(rng.integers(1, 4000))
    w = list(rng.lognormal(0.0, 1.0, L))
    ks = budget.weighted_budgets(w, avg)
    assert sum(ks) == L * avg
    # within one of the real-valued share, and ordered like the weights
    for wl, kl in zip(w, ks):
        assert abs(kl - L * avg * wl / sum(w)) < 1.0 + 1e-9
    for a in range(L):
        for b in range(L):
            if w[a] > w[b]:
                assert ks[a] >= ks[b]
    # a power-of-two scale of every weight changes nothing (exact in binary)
    assert budget.weighted_budgets([x * 8.0 for x in w], avg) == ks


def test_weighted_layer_budgets_cap():
    assert budget.weighted_layer_budgets([1.0, 9.0], 100, prompt_len=150, window=20) == [20, 130]


@pytest.mark.parametrize("name,bits", [("llama3_8b", 2), ("llama3_8b", 4), ("mistral_pyramid", 2),
                                       ("long_context", 2), ("long_context", 4)])
def test_layout_bytes_equal_the_built_cache(name, bits):
    """footprint()['bytes_layout'] with a residual and with eviction equals the
    bytes of the arrays oracle.quant.build_head_cache returns for each layer's
    kept tokens (T = budget + W), summed over layers, times the KV heads: the
    packed codes, the fp16 scale/zero words and the bf16 residual of the
    blog's accounting ("The budget"), laid out as quant.py states."""
    import synth
    from oracle import quant

    cfg = synth.CONFIGS[name]
    L, Hkv, D, n, W, R = cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.prompt, cfg.window, cfg.residual
    fp = budget.footprint(L, Hkv, D, n, W, 0, cfg.budget, cfg.pyramid, cfg.beta, bits, 32, 16, R)
    rng = np.random.default_rng(5)
    total = 0
    for k in budget.layer_budgets(L, cfg.budget, cfg.pyramid, cfg.beta, n, W):
        T = k + W
        x = rng.standard_normal((T, D)).astype(np.float32)
        c = quant.build_head_cache(x, x, np.arange(T), R, bits)
        total += sum(c[key].nbytes for key in ("k_codes", "k_meta", "v_codes", "v_meta", "k_res", "v_res"))
    assert fp["bytes_layout"] == float(total * Hkv)
