"""Full-size parity: every workload at its real shape, through the C ABI, in the
launch configuration the benchmark times (same sizes, capacities and calls).

Every (batch row, KV head) unit is compared:
  * selection: idx equals the oracle's top-k of the GPU's own pooled scores for
    every unit (bit-exact), the scores match the oracle's window scores and the
    kept set matches the oracle's up to near-ties;
  * quantization: the packed cache of every unit is bit-exact against the
    oracle run on the GPU's indices, after the prefill, after every flush and
    after the last step;
  * decode: every unit's outputs against the oracle stepping its own
    (bit-identical) cache, on every step where the cache is small, else on the
    first step, every flush step and the last step (the oracle appends and
    flushes on every step either way).
The oracle's per-unit work runs in a thread pool (numpy releases the GIL in
its array operations).
"""

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import synth
from oracle import decode as odecode
from oracle import quant as oquant
from oracle import select as oselect
import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    ("llama3_8b", 2, 0),
    ("llama3_8b", 2, 0, 16),   # MiniKV's group size
    ("llama3_8b", 2, 0, 32, True),   # MiniKV's whole-residual policy
    ("mistral_pyramid", 2, 0),
    ("mistral_pyramid", 2, 31),
    ("llama2_13b_mha", 4, 0),
    ("llama2_13b_mha", 2, 0),
    ("long_context", 2, 0),
    ("long_context", 2, 31),
]

# oracle attention on every step when units x cached tokens stays below this
EVERY_STEP_TOKENS = 1 << 20
_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def pmap(fn, items):
    return list(_POOL.map(fn, items))


def _units(cfg):
    return [(b, j) for b in range(cfg.batch) for j in range(cfg.kv_heads)]


def compare_all_caches(cache, ref, where):
    """Every unit's packed cache and residual, bit-exact."""
    allc = gu.gpu_all_caches(cache)
    for (b, j), r in ref.items():
        gu.assert_cache_equal(gu.unit_cache(allc, b, j), r, f"{where} b{b} j{j}")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_fullsize_workload(case):
    name, bits, layer = case[:3]
    group = case[3] if len(case) > 3 else 32
    flush_all = case[4] if len(case) > 4 else False
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    cfg = synth.CONFIGS[name]
    B, Hq, Hkv, D, n, W, R = cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.prompt, cfg.window, cfg.residual
    G = cfg.group
    budgets, _ = kvc.kvc_budget(cfg.layers, Hkv, D, n, W, cfg.decode_steps, cfg.budget, cfg.pyramid, cfg.beta,
                                bits=bits, group=32, meta_bits=16, residual=R)
    kb = budgets[layer]
    print(f"[fullsize] {name} layer {layer} bits {bits} group {group} flush_all {flush_all} budget {kb}", flush=True)
    p = synth.prompt_layer(cfg, layer, "cuda")
    units = _units(cfg)

    # ---- selection
    idx = None
    if cfg.budget >= 0:
        idx, scores = kvc.kvc_select(p["q_win"], p["k"], W, cfg.pool, kb, want_scores=True)
        torch.cuda.synchronize()
        sc, ix = scores.cpu().numpy(), idx.cpu().numpy()
        for b, j in units:
            np.testing.assert_array_equal(ix[b, j], oselect.top_k(sc[b, j], ix.shape[-1]), f"b{b} j{j}")
        qw_all, k_all = gu.as_f32(p["q_win"]), gu.as_f32(p["k"])

        def pooled_of(u):
            b, j = u
            qw, kh = qw_all[b:b + 1, j * G:(j + 1) * G], k_all[b:b + 1, j:j + 1]
            return oselect.max_pool(oselect.window_scores(qw, kh, W), cfg.pool)[0, 0]

        swaps = 0
        for (b, j), pooled in zip(units, pmap(pooled_of, units)):
            swaps += gu.check_selection(ix[b, j], sc[b, j], pooled, kb)
        del k_all
        print(f"[fullsize] selection: {len(units)} units exact on own scores and against oracle scores "
              f"({swaps} near-tie swaps)", flush=True)

    # ---- quantization, in the benchmark's capacities
    T = kb + W if cfg.budget >= 0 else n
    r0 = (T % group) if flush_all else None
    nsteps = cfg.decode_steps
    if flush_all:
        nsteps = max(nsteps, R - r0 + 1)  # reach the whole-residual flush and one step past it
    cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=T + nsteps + R + 32, device="cuda", group=group,
                      flush_all=flush_all)
    kvc.kvc_quantize(p["k"], p["v"], cache, idx=idx, W=W)
    torch.cuda.synchronize()
    kf, vf = gu.as_f32(p["k"]), gu.as_f32(p["v"])
    ixc = idx.cpu().numpy() if idx is not None else None
    del p

    def build(u):
        b, j = u
        kept = oquant.kept_positions(n, W, ixc[b, j] if ixc is not None else None)
        return oquant.build_head_cache(kf[b, j], vf[b, j], kept, R, bits, group, flush_all=flush_all)

    ref = dict(zip(units, pmap(build, units)))
    del kf, vf
    compare_all_caches(cache, ref, "prefill")
    print(f"[fullsize] prefill: {len(units)} unit caches bit-exact (q_len {cache.q_len}, r_len {cache.r_len})",
          flush=True)

    # ---- decode: the whole decode run on this layer, every unit
    r_first = cache.r_len
    every = len(units) * (T + nsteps) <= EVERY_STEP_TOKENS
    flushes, compared, worst = 0, 0, 0.0
    for s in range(nsteps):
        d = synth.decode_inputs(cfg, layer, s, "cuda")
        ql = cache.q_len
        out = kvc.kvc_decode_attn(cache, d["q"], d["k_new"], d["v_new"]).cpu().numpy()
        flushed = cache.q_len != ql
        flushes += flushed
        qf = gu.as_f32(d["q"]).astype(np.float64)
        knb, vnb = gu.bf16_bits(d["k_new"]), gu.bf16_bits(d["v_new"])
        check = every or s == 0 or flushed or s == nsteps - 1

        def step(u):
            b, j = u
            if not check:
                return None, oquant.append_and_flush(ref[u], knb[b, j], vnb[b, j], R, bits)
            o_ref, (c,) = odecode.decode_step([ref[u]], qf[b, j * G:(j + 1) * G], knb[b, j:j + 1],
                                              vnb[b, j:j + 1], R, bits)
            return o_ref, c

        res = pmap(step, units)
        for u, (o_ref, c) in zip(units, res):
            ref[u] = c
            if o_ref is not None:
                b, j = u
                err = gu.assert_decode_close(out[b, j * G:(j + 1) * G], o_ref, f"step {s} b{b} j{j}")
                worst = max(worst, err / max(1.0, float(np.abs(o_ref).max())))
        compared += check
        if check and not every:
            print(f"[fullsize] step {s}: {len(units)} units compared", flush=True)
        if flushed:
            torch.cuda.synchronize()
            compare_all_caches(cache, ref, f"flush at step {s}")
    torch.cuda.synchronize()
    compare_all_caches(cache, ref, "after decode")
    # a flush is due once the residual reaches R+g (R with the whole-residual policy)
    if nsteps >= (R if flush_all else R + group) - r_first:
        assert flushes >= 1, "the decode run should have flushed"
    print(f"[fullsize] {name} layer {layer}: {len(units)} units, q_len {cache.q_len} r_len {cache.r_len}, "
          f"{flushes} flushes, outputs compared on {compared}/{nsteps} steps, "
          f"worst normalized decode error {worst:.2e}", flush=True)


def test_split_count_independence():
    """The same head's cache decoded alone (one unit: the planner splits its
    history over many workgroups) and replicated over 128 units (few splits per
    unit): every output equals the oracle's within the decode bound, and the
    two launch shapes agree with each other to float32 rounding (MiniKV Eq. 1:
    one output per query head, whatever the split of the token range)."""
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    n, D, R, bits = 16384, 128, 128, 2
    k1, v1 = synth.random_case(11, 1, 4, 1, D, n, "bf16", "cuda", key_scale=2.0)
    q1 = synth.random_tensor(12, (1, 4, D), "bf16", "cuda", tag="split-q")
    kn1 = synth.random_tensor(13, (1, 1, D), "bf16", "cuda", tag="split-k")
    vn1 = synth.random_tensor(14, (1, 1, D), "bf16", "cuda", tag="split-v")
    outs = {}
    for B, Hkv in ((1, 1), (16, 8)):
        k = k1.expand(B, Hkv, n, D).contiguous()
        v = v1.expand(B, Hkv, n, D).contiguous()
        q = q1.reshape(1, 1, 4, D).expand(B, Hkv, 4, D).reshape(B, Hkv * 4, D).contiguous()
        kn = kn1.expand(B, Hkv, D).contiguous()
        vn = vn1.expand(B, Hkv, D).contiguous()
        cache = kvc.Cache(B, Hkv, D, bits, R, q_cap=n + 64, device="cuda")
        kvc.kvc_quantize(k, v, cache)
        outs[(B, Hkv)] = kvc.kvc_decode_attn(cache, q, kn, vn).cpu().numpy().reshape(B, Hkv, 4, D)
        del k, v, cache
    ref = oquant.build_head_cache(gu.as_f32(k1[0, 0]), gu.as_f32(v1[0, 0]), np.arange(n), R, bits)
    o_ref, _ = odecode.decode_step([ref], gu.as_f32(q1[0]).astype(np.float64), gu.bf16_bits(kn1[0]),
                                   gu.bf16_bits(vn1[0]), R, bits)
    one = outs[(1, 1)][0, 0]
    gu.assert_decode_close(one, o_ref, "one unit")
    many = outs[(16, 8)]
    for b in range(16):
        for j in range(8):
            gu.assert_decode_close(many[b, j], o_ref, f"replica b{b} j{j}")
            np.testing.assert_allclose(many[b, j], one, rtol=0, atol=2e-5 * max(1.0, float(np.abs(one).max())))


@pytest.mark.parametrize("name,layer", [("llama3_8b", 0), ("long_context", 0)])
def test_fullsize_variance_budget_path(name, layer):
    """Prompt compression of the variance budget policies at full size, in the
    calls the benchmark makes for them: kvc_window_scores (raw window scores and
    their variance per head), then kvc_topk at the layer's budget.  Every head:
    the variance against the oracle's on the GPU's own scores, the pooled scores
    and indices exact on those scores, the same indices as kvc_select, and the
    raw scores against the oracle's window scores."""
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    cfg = synth.CONFIGS[name]
    B, Hkv, D, n, W, G = cfg.batch, cfg.kv_heads, cfg.head_dim, cfg.prompt, cfg.window, cfg.group
    budgets, _ = kvc.kvc_budget(cfg.layers, Hkv, D, n, W, cfg.decode_steps, cfg.budget, cfg.pyramid, cfg.beta,
                                bits=cfg.bits[0], group=32, meta_bits=16, residual=cfg.residual)
    kb = budgets[layer]
    print(f"[fullsize] variance path {name} layer {layer} budget {kb}", flush=True)
    p = synth.prompt_layer(cfg, layer, "cuda")
    raw, var = kvc.kvc_window_scores(p["q_win"], p["k"], W)
    idx, pooled = kvc.kvc_topk(raw, cfg.pool, kb, want_scores=True)
    idx_fused = kvc.kvc_select(p["q_win"], p["k"], W, cfg.pool, kb)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_fused)
    r, v, pc, ix = raw.cpu().numpy(), var.cpu().numpy(), pooled.cpu().numpy(), idx.cpu().numpy()
    np.testing.assert_allclose(v, oselect.score_variance(r), rtol=1e-6)
    np.testing.assert_array_equal(pc, oselect.max_pool(r.astype(np.float64), cfg.pool).astype(np.float32))
    for b in range(B):
        for j in range(Hkv):
            np.testing.assert_array_equal(ix[b, j], oselect.top_k(pc[b, j], ix.shape[-1]), f"b{b} j{j}")
    qw_all, k_all = gu.as_f32(p["q_win"]), gu.as_f32(p["k"])

    def raw_of(u):
        b, j = u
        return oselect.window_scores(qw_all[b:b + 1, j * G:(j + 1) * G], k_all[b:b + 1, j:j + 1], W)[0, 0]

    units = _units(cfg)
    for (b, j), ref in zip(units, pmap(raw_of, units)):
        np.testing.assert_array_less(np.abs(r[b, j] - ref), gu.SCORE_TOL * (np.abs(ref) + ref.max()) + 1e-30)
