"""GPU parity of each stage, through the C ABI, against the oracle on the same
seeded inputs: bit-exact codes, scales, residual and indices; decode outputs
within 2e-3.  Sizes span several tiles with ragged tails."""

import numpy as np
import pytest
import torch

import synth
from oracle import decode as odecode
from oracle import quant as oquant
from oracle import select as oselect
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _kvc():
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc
    return kvc


def _case(seed, B, Hkv, n, D, dtype, outliers=True):
    scale = None
    if outliers:
        g = torch.Generator().manual_seed(seed)
        scale = torch.exp(0.5 * torch.randn(D, generator=g))
        scale[torch.randperm(D, generator=g)[:2]] *= 8
    k, v = synth.random_case(seed, B, Hkv, Hkv, D, n, dtype, key_scale=scale)
    return k.cuda(), v.cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("D", [64, 96, 128, 224])   # 96, 224: head dims below the LDS layout's bound
@pytest.mark.parametrize("with_idx", [True, False])
def test_quantize_parity(dtype, bits, D, with_idx):
    kvc = _kvc()
    B, Hkv, n, W, R = 2, 3, 300, 8, 16
    k, v = _case(1, B, Hkv, n, D, dtype)
    idx = None
    k_sel = 0
    if with_idx:
        g = torch.Generator().manual_seed(2)
        k_sel = 100
        idx = torch.stack([torch.stack([torch.sort(torch.randperm(n - W, generator=g)[:k_sel]).values
                                        for _ in range(Hkv)]) for _ in range(B)]).to(torch.int32).cuda()
    T = k_sel + W if with_idx else n
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=T + 64, device="cuda")
    kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
    torch.cuda.synchronize()
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    for b in range(B):
        for j in range(Hkv):
            kept = oquant.kept_positions(n, W, idx[b, j].cpu().numpy() if with_idx else None)
            ref = oquant.build_head_cache(kf[b, j], vf[b, j], kept, R, bits)
            gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref, f"b{b} j{j}")


def _degenerate_case(dtype, n, D, group):
    """Random keys and values with degenerate groups planted in the first key
    group and in value tokens 5..9 (MiniKV Sec. 4.4 fp16 scale/zero): constant
    groups (zero scale), ranges too wide for fp16 (infinite scale), ranges too
    small for it (scale 0 after rounding), and groups near +-1e5 whose fp16 zero
    overflows while the scale stays finite (t = +-inf, codes clamp)."""
    g = torch.Generator().manual_seed(21)
    k = torch.randn(1, 2, n, D, generator=g)
    v = torch.randn(1, 2, n, D, generator=g)
    r = torch.rand(group, generator=g)
    k[:, :, :group, 0:4] = 0.75                                         # constant
    k[:, :, :group, 4] = torch.where(torch.arange(group) % 2 == 0, 1e6, -1e6)  # inf scale, -inf zero
    k[:, :, :group, 5] = 4e6 * r                                        # inf scale, finite zero
    k[:, :, 0, 5] = 0.0
    k[:, :, :group, 6] = 1e-30 * (r - 0.5)                              # scale and zero underflow
    k[:, :, :group, 7] = -1e5 + 4000 * r                                 # -inf zero, finite scale
    k[:, :, :group, 8] = 99000 + 4000 * r                                # +inf zero, finite scale
    v[:, :, 5, :] = 2.5
    v[:, :, 6, :] = torch.where(torch.arange(D) % 3 == 0, 1e6, -1e6)
    v[:, :, 7, :] = 1e-30 * torch.randn(D, generator=g)
    v[:, :, 8, :] = -1e5 + 4000 * torch.rand(D, generator=g)
    v[:, :, 9, :] = 99000 + 4000 * torch.rand(D, generator=g)
    if dtype == "bf16":
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    return k.cuda(), v.cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("group", [32, 16])
def test_quantize_degenerate_groups(dtype, bits, group):
    """Groups whose scale is zero, overflows or underflows fp16, or whose zero
    overflows: codes and metadata bit-exact against the oracle (all-zero codes
    where the scale is zero or not finite, clamped codes where t is infinite)."""
    kvc = _kvc()
    n, D, R = 160, 64, 16
    k, v = _degenerate_case(dtype, n, D, group)
    cache = kvc.Cache(1, 2, D, bits, R, q_cap=n + 64, device="cuda", group=group)
    kvc.kvc_quantize(k, v, cache)
    torch.cuda.synchronize()
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    for j in range(2):
        ref = oquant.build_head_cache(kf[0, j], vf[0, j], np.arange(n), R, bits, group)
        gu.assert_cache_equal(gu.gpu_head_cache(cache, 0, j), ref, f"j{j}")
        # the planted groups really are degenerate in the oracle
        s_bits = (ref["k_meta"][0, :9] & 0xFFFF).astype(np.uint16).view(np.float16)
        assert (s_bits[:4] == 0).all() and np.isinf(s_bits[4:6]).all() and s_bits[6] == 0
        z_bits = (ref["k_meta"][0, 7:9] >> 16).astype(np.uint16).view(np.float16)
        assert np.isinf(z_bits).all() and np.isfinite(s_bits[7:9]).all()


@pytest.mark.parametrize("dtype,bits,G,D,R,n", [
    ("bf16", 2, 4, 128, 16, 300), ("bf16", 4, 1, 128, 16, 300), ("f32", 2, 1, 64, 16, 250),
    ("bf16", 2, 2, 64, 0, 200), ("bf16", 4, 8, 32, 40, 160), ("f32", 4, 3, 256, 24, 130),
    ("bf16", 2, 16, 64, 16, 100),
    # histories long enough for the split runs (several workgroups per unit, merged)
    ("f32", 2, 1, 128, 16, 3000), ("f32", 4, 4, 128, 128, 2600), ("bf16", 2, 4, 128, 128, 4000),
    ("bf16", 2, 4, 256, 16, 3000),   # D = 256: four heads per workgroup in the split runs
    # odd multiples of 32 (three, five and seven key slices per lane group), short and split runs
    ("bf16", 2, 2, 96, 16, 300), ("f32", 4, 1, 160, 24, 200), ("bf16", 2, 4, 224, 16, 2600)])
def test_decode_parity_multi_step(dtype, bits, G, D, R, n):
    kvc = _kvc()
    B, Hkv = 2, 2
    Hq = Hkv * G
    steps = 40
    k, v = _case(3, B, Hkv, n, D, dtype)
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=n + steps + 32, device="cuda")
    kvc.kvc_quantize(k, v, cache)
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    ref = [[oquant.build_head_cache(kf[b, j], vf[b, j], np.arange(n), R, bits) for j in range(Hkv)]
           for b in range(B)]
    worst = 0.0
    flushes = 0
    for s in range(steps):
        q = synth.random_tensor(100 + s, (B, Hq, D), dtype, tag="q").cuda()
        kn = synth.random_tensor(200 + s, (B, Hkv, D), dtype, tag="kn").cuda()
        vn = synth.random_tensor(300 + s, (B, Hkv, D), dtype, tag="vn").cuda()
        ql = cache.q_len
        out = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy()
        flushes += cache.q_len != ql
        qf = gu.as_f32(q).astype(np.float64)
        knb, vnb = gu.bf16_bits(kn), gu.bf16_bits(vn)
        for b in range(B):
            o_ref, ref[b] = odecode.decode_step(ref[b], qf[b], knb[b], vnb[b], R, bits)
            worst = max(worst, gu.assert_decode_close(out[b], o_ref, f"step {s} b{b}"))
    torch.cuda.synchronize()
    for b in range(B):
        for j in range(Hkv):
            gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref[b][j], f"after steps b{b} j{j}")
    assert flushes >= 1


@pytest.mark.parametrize("dtype,B,G,Hkv,n,D,W,pool,budget", [
    ("bf16", 2, 4, 2, 700, 128, 16, 7, 100), ("f32", 1, 1, 4, 512, 64, 8, 5, 64),
    ("bf16", 1, 2, 3, 333, 64, 5, 3, 40), ("bf16", 1, 8, 1, 1000, 256, 32, 7, 200),
    ("f32", 2, 3, 1, 257, 32, 13, 1, 30), ("bf16", 1, 4, 2, 300, 128, 300, 7, 10),
    ("bf16", 1, 4, 2, 300, 128, 20, 7, 0), ("bf16", 1, 4, 2, 300, 128, 20, 7, 5000),
    ("bf16", 1, 4, 2, 300, 128, 20, 7, -1), ("bf16", 1, 1, 1, 2000, 128, 150, 9, 333),
    ("bf16", 2, 2, 2, 600, 32, 24, 5, 80), ("bf16", 1, 16, 1, 900, 64, 16, 7, 100),
    # odd numbers of 32-channel slices (the general scorer)
    ("bf16", 1, 4, 2, 500, 96, 16, 7, 60), ("f32", 1, 2, 1, 400, 160, 12, 5, 50),
    ("bf16", 1, 2, 1, 700, 224, 24, 7, 90),
    # rows of 9k-32k candidates (keys in registers, raw scores in LDS)
    ("bf16", 1, 2, 1, 12000, 64, 16, 7, 900), ("bf16", 1, 1, 1, 30000, 64, 8, 7, 2000),
    # rows above 32k candidates: 4096-candidate chunks over many workgroups
    ("bf16", 1, 2, 2, 40000, 64, 16, 7, 1500), ("f32", 1, 1, 1, 36000, 32, 8, 13, 700),
    ("bf16", 1, 1, 2, 34000, 64, 8, 3, -1), ("bf16", 1, 1, 1, 34000, 64, 8, 5, 0)])
def test_select_parity(dtype, B, G, Hkv, n, D, W, pool, budget):
    kvc = _kvc()
    Hq = G * Hkv
    k, _ = _case(5, B, Hkv, n, D, dtype)
    q_win = synth.random_tensor(6, (B, Hq, W, D), dtype, tag="qw").cuda()
    idx, scores = kvc.kvc_select(q_win, k, W, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    N = n - W
    assert idx.shape == (B, Hkv, N if budget < 0 else min(budget, N))
    if N == 0:
        return
    pooled = oselect.max_pool(oselect.window_scores(gu.as_f32(q_win), gu.as_f32(k), W), pool)
    sc = scores.cpu().numpy()
    ix = idx.cpu().numpy()
    for b in range(B):
        for j in range(Hkv):
            gu.check_selection(ix[b, j], sc[b, j], pooled[b, j], budget)


@pytest.mark.parametrize("dtype,B,G,Hkv,n,D,W,pool,budget", [
    ("bf16", 2, 4, 2, 700, 128, 16, 7, 100), ("f32", 1, 1, 4, 512, 64, 8, 5, 64),
    ("bf16", 1, 8, 1, 1000, 128, 32, 7, 200),     # 256 window rows
    ("bf16", 1, 3, 2, 333, 32, 5, 3, 40),
    ("bf16", 1, 2, 2, 40000, 64, 16, 7, 1500)])   # rows above 32k candidates
def test_select_lse_parity(dtype, B, G, Hkv, n, D, W, pool, budget):
    """kvc_select_lse with the window rows' log-sum-exp from kvc_prefill_attn
    (the prompt's own prefill, its last W query rows being q_win): the scores
    and indices meet the same checks against the oracle as kvc_select's."""
    kvc = _kvc()
    Hq = G * Hkv
    k, v = _case(21, B, Hkv, n, D, dtype)
    q = synth.random_tensor(22, (B, Hq, n, D), dtype, tag="q").cuda()
    q_win = q[:, :, n - W:].contiguous()
    lse = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
    kvc.kvc_prefill_attn(q, k, v, want_acc=False, lse=lse)
    idx, scores = kvc.kvc_select_lse(q_win, k, lse, W, pool, budget, want_scores=True)
    idx2, _ = kvc.kvc_select_lse(q_win, k, lse[:, :, n - W:].contiguous(), W, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)  # a compact [B][Hq][W] lse gives the same selection
    pooled = oselect.max_pool(oselect.window_scores(gu.as_f32(q_win), gu.as_f32(k), W), pool)
    sc, ix = scores.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        for j in range(Hkv):
            gu.check_selection(ix[b, j], sc[b, j], pooled[b, j], budget)


@pytest.mark.parametrize("budget", [-1, 280, 5000])
def test_select_keep_all_without_scores(budget):
    """Keeping every candidate needs no ranking: without scores kvc_select
    writes 0..n-W-1 per (b, KV head) (no scorer launch), the same idx as the
    scored call; a smaller budget still ranks."""
    kvc = _kvc()
    B, G, Hkv, n, D, W = 2, 4, 2, 300, 128, 20
    k, _ = _case(8, B, Hkv, n, D, "bf16")
    q_win = synth.random_tensor(9, (B, G * Hkv, W, D), "bf16", tag="qw").cuda()
    idx = kvc.kvc_select(q_win, k, W, 7, budget)
    idx_s, _ = kvc.kvc_select(q_win, k, W, 7, budget, want_scores=True)
    torch.cuda.synchronize()
    want = torch.arange(n - W, dtype=torch.int32).expand(B, Hkv, n - W)
    assert torch.equal(idx.cpu(), want) and torch.equal(idx_s.cpu(), want)
    idx2 = kvc.kvc_select(q_win, k, W, 7, n - W - 1)
    idx2_s, _ = kvc.kvc_select(q_win, k, W, 7, n - W - 1, want_scores=True)
    torch.cuda.synchronize()
    assert idx2.shape == (B, Hkv, n - W - 1) and torch.equal(idx2.cpu(), idx2_s.cpu())


@pytest.mark.parametrize("dtype,B,G,Hkv,n,D,W", [
    ("bf16", 2, 4, 2, 700, 128, 16), ("f32", 1, 1, 3, 300, 64, 8), ("bf16", 1, 8, 1, 1000, 256, 32),
    ("bf16", 1, 4, 1, 2000, 128, 64), ("bf16", 1, 2, 2, 37000, 64, 16)])
def test_window_scores_and_variance(dtype, B, G, Hkv, n, D, W):
    """kvc_window_scores: raw column sums against the oracle's window scores, and
    their variance (MiniKV's variance score) against the oracle's, on the GPU's
    own scores (float64 accumulation: tight) and on the oracle's scores."""
    kvc = _kvc()
    k, _ = _case(15, B, Hkv, n, D, dtype)
    q_win = synth.random_tensor(16, (B, Hkv * G, W, D), dtype, tag="qw").cuda()
    raw, var = kvc.kvc_window_scores(q_win, k, W)
    torch.cuda.synchronize()
    ref = oselect.window_scores(gu.as_f32(q_win), gu.as_f32(k), W)
    r = raw.cpu().numpy()
    np.testing.assert_array_less(np.abs(r - ref), gu.SCORE_TOL * (np.abs(ref) + ref.max()) + 1e-30)
    v = var.cpu().numpy()
    np.testing.assert_allclose(v, oselect.score_variance(r), rtol=1e-5)
    np.testing.assert_allclose(v, oselect.score_variance(ref), rtol=1e-3)
    # the fused call selects the same positions as the two halves
    idx = kvc.kvc_select(q_win, k, W, 7, 100)
    idx2 = kvc.kvc_topk(raw, 7, 100)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("B,Hkv,N,pool,budget", [
    (2, 3, 500, 7, 100), (1, 2, 40000, 7, 1500), (1, 1, 33000, 13, 700), (2, 2, 1000, 1, -1),
    (1, 2, 300, 5, 0), (1, 1, 8160, 9, 512), (3, 1, 4096 * 9, 3, 1),
    # rows shorter than a pooling window and than one thread's candidates (the
    # padded LDS row), and rows that end inside the last thread's candidates
    (1, 1, 1, 7, 1), (2, 1, 5, 9, 2), (1, 2, 9, 3, 4), (1, 1, 8195, 7, 600), (1, 1, 16390, 5, 1000)])
def test_topk_on_given_scores(B, Hkv, N, pool, budget):
    """kvc_topk on seeded scores on a coarse grid (many ties): the pooled scores
    are maxima of the inputs (exact) and idx is the oracle's top-k of them."""
    kvc = _kvc()
    raw = (torch.round(synth.random_tensor(17, (B, Hkv, N), "f32", tag="raw") * 8) / 8).cuda()
    idx, sc = kvc.kvc_topk(raw, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    pooled = oselect.max_pool(raw.cpu().numpy().astype(np.float64), pool)
    np.testing.assert_array_equal(sc.cpu().numpy(), pooled.astype(np.float32))
    kk = N if budget < 0 else min(budget, N)
    ix = idx.cpu().numpy()
    assert ix.shape == (B, Hkv, kk)
    for b in range(B):
        for j in range(Hkv):
            np.testing.assert_array_equal(ix[b, j], oselect.top_k(pooled[b, j], kk), f"b{b} j{j}")


@pytest.mark.parametrize("n", [3000, 40000])
def test_select_all_scores_tied(n):
    """Zero keys make every logit 0, so every candidate gets the same score (the
    same terms summed in the same order) and the top-k is the k lowest
    positions; with 40000 the tie spans every chunk of the long-row path."""
    kvc = _kvc()
    B, Hkv, G, D, W, pool, budget = 1, 2, 2, 64, 16, 7, 1234
    k = torch.zeros(B, Hkv, n, D, dtype=torch.bfloat16, device="cuda")
    q_win = synth.random_tensor(7, (B, Hkv * G, W, D), "bf16", tag="qw").cuda()
    idx, scores = kvc.kvc_select(q_win, k, W, pool, budget, want_scores=True)
    torch.cuda.synchronize()
    sc = scores.cpu()
    assert torch.equal(sc, sc[:, :, :1].expand_as(sc)), "scores not all equal"
    want = torch.arange(budget, dtype=torch.int32).expand(B, Hkv, budget)
    assert torch.equal(idx.cpu(), want)


def test_select_planted_and_dense_special_case():
    """Budget >= n-W keeps everything and the step equals dense attention."""
    kvc = _kvc()
    B, Hkv, G, n, D, W = 1, 2, 2, 200, 64, 8
    k, v = _case(9, B, Hkv, n, D, "bf16")
    q_win = synth.random_tensor(10, (B, Hkv * G, W, D), "bf16", tag="qw").cuda()
    idx = kvc.kvc_select(q_win, k, W, 5, n)
    assert torch.equal(idx[0, 0].cpu(), torch.arange(n - W, dtype=torch.int32))
    cache = kvc.Cache(B, Hkv, D, 2, residual=n + 1, q_cap=32, r_cap=n + 64, device="cuda")
    kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
    assert cache.q_len == 0 and cache.r_len == n
    q = synth.random_tensor(11, (B, Hkv * G, D), "bf16", tag="q").cuda()
    kn = synth.random_tensor(12, (B, Hkv, D), "bf16", tag="kn").cuda()
    vn = synth.random_tensor(13, (B, Hkv, D), "bf16", tag="vn").cuda()
    out = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy()
    K = torch.cat([k, kn[:, :, None]], 2).double().cpu().repeat_interleave(G, 1)
    V = torch.cat([v, vn[:, :, None]], 2).double().cpu().repeat_interleave(G, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double().cpu()[:, :, None], K, V)[:, :, 0]
    gu.assert_decode_close(out[0], ref[0].numpy(), "dense")


def test_tiny_config_end_to_end():
    """The tiny workload through all stages, stage-wise and end to end."""
    kvc = _kvc()
    cfg = synth.CONFIGS["tiny"]
    p = synth.prompt_layer(cfg, 0, "cpu")
    d = synth.decode_inputs(cfg, 0, 0, "cpu")
    q_win, k, v = p["q_win"].cuda(), p["k"].cuda(), p["v"].cuda()
    idx, scores = kvc.kvc_select(q_win, k, cfg.window, cfg.pool, cfg.budget, want_scores=True)
    bits = cfg.bits[0]
    T = cfg.budget + cfg.window
    cache = kvc.Cache(cfg.batch, cfg.kv_heads, cfg.head_dim, bits, cfg.residual, q_cap=T + 32, device="cuda")
    kvc.kvc_quantize(k, v, cache, idx=idx, W=cfg.window)
    out = kvc.kvc_decode_attn(cache, d["q"].cuda(), d["k_new"].cuda(), d["v_new"].cuda()).cpu().numpy()
    assert (cache.q_len, cache.r_len) == (32, 41)
    qw, kf, vf = gu.as_f32(p["q_win"]), gu.as_f32(p["k"]), gu.as_f32(p["v"])
    oidx, pooled = oselect.select(qw, kf, cfg.window, cfg.pool, cfg.budget)
    swaps = gu.check_selection(idx[0, 0].cpu().numpy(), scores[0, 0].cpu().numpy(), pooled[0, 0], cfg.budget)
    for j in range(1, cfg.kv_heads):
        swaps += gu.check_selection(idx[0, j].cpu().numpy(), scores[0, j].cpu().numpy(), pooled[0, j], cfg.budget)
    assert swaps == 0
    n, W = cfg.prompt, cfg.window
    ref = [oquant.build_head_cache(kf[0, j], vf[0, j], oquant.kept_positions(n, W, oidx[0, j]),
                                   cfg.residual, bits) for j in range(cfg.kv_heads)]
    qf = gu.as_f32(d["q"]).astype(np.float64)
    o_ref, ref = odecode.decode_step(ref, qf[0], gu.bf16_bits(d["k_new"])[0], gu.bf16_bits(d["v_new"])[0],
                                     cfg.residual, bits)
    for j in range(cfg.kv_heads):
        gu.assert_cache_equal(gu.gpu_head_cache(cache, 0, j), ref[j], f"j{j}")
    gu.assert_decode_close(out[0], o_ref, "tiny end-to-end")


@pytest.mark.parametrize("B,Hkv,n,W,budget,sinks", [
    (2, 3, 300, 8, 100, 4), (2, 2, 300, 8, 100, 0), (1, 1, 50, 10, 100, 4), (2, 2, 300, 8, -1, 7),
    (2, 2, 300, 8, 5, 9), (3, 2, 64, 64, 10, 4), (2, 2, 300, 8, 0, 4),
    (8, 8, 40000, 32, 20000, 4)])   # 1.28M entries: several grid-stride passes
def test_select_recent_parity(B, Hkv, n, W, budget, sinks):
    kvc = _kvc()
    idx = kvc.kvc_select_recent(B, Hkv, n, W, budget, sinks)
    torch.cuda.synchronize()
    want = torch.from_numpy(oselect.recent_select(n, W, budget, sinks))
    assert tuple(idx.shape) == (B, Hkv, len(want))
    assert torch.equal(idx.cpu(), want.expand(B, Hkv, -1))


def test_recent_selection_end_to_end():
    """Sinks + recent window through quantize and two decode steps (with the
    appended tokens), against the oracle on the same kept positions."""
    kvc = _kvc()
    B, Hkv, G, D, n, W, budget, sinks, bits, R = 2, 2, 4, 128, 500, 16, 150, 4, 2, 32
    k, v = _case(41, B, Hkv, n, D, "bf16")
    idx = kvc.kvc_select_recent(B, Hkv, n, W, budget, sinks)
    T = budget + W
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=T + 64, device="cuda")
    kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    kept = oquant.kept_positions(n, W, oselect.recent_select(n, W, budget, sinks))
    assert list(kept[:sinks]) == list(range(sinks)) and list(kept[sinks:]) == list(range(n - (T - sinks), n))
    ref = [[oquant.build_head_cache(kf[b, j], vf[b, j], kept, R, bits) for j in range(Hkv)] for b in range(B)]
    for s in range(2):
        q = synth.random_tensor(300 + s, (B, Hkv * G, D), "bf16", tag="q").cuda()
        kn = synth.random_tensor(400 + s, (B, Hkv, D), "bf16", tag="kn").cuda()
        vn = synth.random_tensor(500 + s, (B, Hkv, D), "bf16", tag="vn").cuda()
        out = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy()
        qf = gu.as_f32(q).astype(np.float64)
        for b in range(B):
            o_ref, ref[b] = odecode.decode_step(ref[b], qf[b], gu.bf16_bits(kn)[b], gu.bf16_bits(vn)[b], R, bits)
            gu.assert_decode_close(out[b], o_ref, f"step {s} b{b}")
            for j in range(Hkv):
                gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref[b][j], f"step {s} b{b} j{j}")


# ---------------------------------------------------------------- group size 16
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("D,with_idx", [(64, True), (128, False), (256, True), (96, True), (224, False)])
def test_quantize_parity_group16(dtype, bits, D, with_idx):
    """MiniKV's group of 16 (keys per channel over 16 tokens, values per token
    over 16 channels): packed codes, metadata and residual bit-exact against the
    oracle, with and without a selection."""
    kvc = _kvc()
    B, Hkv, n, W, R = 2, 2, 300, 8, 16
    k, v = _case(11, B, Hkv, n, D, dtype)
    idx, k_sel = None, 0
    if with_idx:
        g = torch.Generator().manual_seed(12)
        k_sel = 123
        idx = torch.stack([torch.stack([torch.sort(torch.randperm(n - W, generator=g)[:k_sel]).values
                                        for _ in range(Hkv)]) for _ in range(B)]).to(torch.int32).cuda()
    T = k_sel + W if with_idx else n
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=T + 64, device="cuda", group=16)
    kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
    torch.cuda.synchronize()
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    for b in range(B):
        for j in range(Hkv):
            kept = oquant.kept_positions(n, W, idx[b, j].cpu().numpy() if with_idx else None)
            ref = oquant.build_head_cache(kf[b, j], vf[b, j], kept, R, bits, 16)
            gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref, f"b{b} j{j}")


@pytest.mark.parametrize("dtype,bits,G,D,R,n", [
    ("bf16", 2, 4, 128, 16, 300), ("bf16", 4, 2, 64, 0, 200), ("f32", 2, 1, 256, 24, 130),
    ("bf16", 4, 8, 32, 40, 160), ("bf16", 2, 2, 128, 128, 700),
    # split runs: one head per workgroup with staged tiles, four heads per
    # workgroup, and f32 inputs; the history alternates between an even and an
    # odd number of 16-token groups (a half-full last tile)
    ("bf16", 2, 1, 128, 16, 4000), ("bf16", 4, 4, 128, 128, 2600), ("f32", 2, 1, 128, 16, 3000),
    ("bf16", 2, 1, 64, 16, 5000),
    ("bf16", 2, 4, 256, 16, 3000),   # D = 256: one head per workgroup (four would not fit a CU's LDS)
    ("bf16", 2, 2, 96, 16, 400), ("f32", 4, 1, 160, 32, 2600)])   # odd numbers of 32-channel slices
def test_decode_parity_group16_multi_step(dtype, bits, G, D, R, n):
    """Decode over group-16 caches for 40 steps (several 16-token flushes, the
    residual ring wrapping): outputs within the decode tolerance and the cache
    bit-exact against the oracle stepping its own cache."""
    kvc = _kvc()
    B, Hkv, steps = 2, 2, 40
    Hq = Hkv * G
    k, v = _case(13, B, Hkv, n, D, dtype)
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=n + steps + 32, device="cuda", group=16)
    kvc.kvc_quantize(k, v, cache)
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    ref = [[oquant.build_head_cache(kf[b, j], vf[b, j], np.arange(n), R, bits, 16) for j in range(Hkv)]
           for b in range(B)]
    flushes = 0
    for s in range(steps):
        q = synth.random_tensor(400 + s, (B, Hq, D), dtype, tag="q").cuda()
        kn = synth.random_tensor(500 + s, (B, Hkv, D), dtype, tag="kn").cuda()
        vn = synth.random_tensor(600 + s, (B, Hkv, D), dtype, tag="vn").cuda()
        ql = cache.q_len
        out = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy()
        flushes += cache.q_len != ql
        qf = gu.as_f32(q).astype(np.float64)
        knb, vnb = gu.bf16_bits(kn), gu.bf16_bits(vn)
        for b in range(B):
            o_ref, ref[b] = odecode.decode_step(ref[b], qf[b], knb[b], vnb[b], R, bits)
            gu.assert_decode_close(out[b], o_ref, f"step {s} b{b}")
    torch.cuda.synchronize()
    for b in range(B):
        for j in range(Hkv):
            gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref[b][j], f"after steps b{b} j{j}")
    assert flushes >= 2


# ---------------------------------------------------------------- whole-residual flush
@pytest.mark.parametrize("group,R,bits,G,D", [(32, 64, 2, 4, 128), (16, 48, 4, 2, 64), (16, 16, 2, 1, 128)])
def test_decode_parity_flush_all(group, R, bits, G, D):
    """MiniKV's whole-residual policy (flush_all): the prefill quantizes every
    complete group, the residual is quantized whole (R/g groups, the appended
    token last) when it reaches R; 100 steps with several such flushes, outputs
    within the decode tolerance and the cache bit-exact against the oracle."""
    kvc = _kvc()
    B, Hkv, n, steps = 2, 2, 300, 100
    Hq = Hkv * G
    k, v = _case(17, B, Hkv, n, D, "bf16")
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=n + steps + 64, device="cuda", group=group, flush_all=True)
    kvc.kvc_quantize(k, v, cache)
    kf, vf = gu.as_f32(k), gu.as_f32(v)
    ref = [[oquant.build_head_cache(kf[b, j], vf[b, j], np.arange(n), R, bits, group, flush_all=True)
            for j in range(Hkv)] for b in range(B)]
    torch.cuda.synchronize()
    for b in range(B):
        for j in range(Hkv):
            gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref[b][j], f"prefill b{b} j{j}")
    flushes = 0
    for s in range(steps):
        q = synth.random_tensor(700 + s, (B, Hq, D), "bf16", tag="q").cuda()
        kn = synth.random_tensor(800 + s, (B, Hkv, D), "bf16", tag="kn").cuda()
        vn = synth.random_tensor(900 + s, (B, Hkv, D), "bf16", tag="vn").cuda()
        ql = cache.q_len
        out = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy()
        flushes += cache.q_len != ql
        qf = gu.as_f32(q).astype(np.float64)
        knb, vnb = gu.bf16_bits(kn), gu.bf16_bits(vn)
        for b in range(B):
            o_ref, ref[b] = odecode.decode_step(ref[b], qf[b], knb[b], vnb[b], R, bits)
            gu.assert_decode_close(out[b], o_ref, f"step {s} b{b}")
        if cache.q_len != ql:
            torch.cuda.synchronize()
            for b in range(B):
                for j in range(Hkv):
                    gu.assert_cache_equal(gu.gpu_head_cache(cache, b, j), ref[b][j], f"flush step {s} b{b} j{j}")
    assert flushes == (n % group + steps) // R >= 1
