"""The whole path captured into one HIP graph (as the benchmark runs it) and
replayed several times, with eager work and synchronizations between replays:
every replay must reproduce the eager run bit for bit (the kernels are
deterministic: no floating-point atomics), including a residual flush."""

import pytest
import torch

import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [32, 16])
def test_graph_replays_equal_eager(group):
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    B, Hkv, G, D, n, W, pool, budget, bits, R, steps = 2, 2, 4, 128, 700, 16, 7, 150, 2, 16, 40
    Hq = Hkv * G
    k, v = synth.random_case(21, B, Hkv, Hkv, D, n, "bf16", device="cuda")
    q_win = synth.random_tensor(22, (B, Hq, W, D), "bf16", tag="qw").cuda()
    dec = [(synth.random_tensor(30 + s, (B, Hq, D), "bf16", tag="q").cuda(),
            synth.random_tensor(130 + s, (B, Hkv, D), "bf16", tag="kn").cuda(),
            synth.random_tensor(230 + s, (B, Hkv, D), "bf16", tag="vn").cuda()) for s in range(steps)]
    T = budget + W

    def make_cache():
        return kvc.Cache(B, Hkv, D, bits, R, q_cap=T + steps + 32, device="cuda", group=group)

    sel_ws = torch.empty(kvc.select_ws_bytes(1, B, Hq, Hkv, n, D, W, pool, budget), dtype=torch.uint8,
                         device="cuda")

    def run(cache, idx, dec_ws, outs):
        cache.reset()
        kvc.kvc_select(q_win, k, W, pool, budget, ws=sel_ws, idx=idx)
        kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
        for s, (q, kn, vn) in enumerate(dec):
            kvc.kvc_decode_attn(cache, q, kn, vn, out=outs[s], ws=dec_ws)

    # eager reference
    c0 = make_cache()
    idx0 = torch.empty(B, Hkv, budget, dtype=torch.int32, device="cuda")
    ws0 = torch.zeros(kvc.decode_ws_bytes(c0, Hq), dtype=torch.uint8, device="cuda")
    outs0 = [torch.empty(B, Hq, D, dtype=torch.float32, device="cuda") for _ in range(steps)]
    run(c0, idx0, ws0, outs0)
    torch.cuda.synchronize()
    assert c0.q_len > group * ((T - R) // group), "the run must include a flush"
    ref = [o.clone() for o in outs0]
    ref_cache = {key: t.clone() for key, t in c0.views().items()}

    # capture the same run
    c1 = make_cache()
    idx1 = torch.empty_like(idx0)
    ws1 = torch.zeros_like(ws0)
    outs1 = [torch.empty_like(o) for o in outs0]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(c1, idx1, ws1, outs1)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs1:
            o.fill_(float("nan"))
        idx1.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx0), f"replay {rep}: idx"
        for s in range(steps):
            assert torch.equal(outs1[s], ref[s]), f"replay {rep}: step {s}"
        for key, t in c1.views().items():
            assert torch.equal(t, ref_cache[key]), f"replay {rep}: {key}"
        # eager work between replays
        run(c0, idx0, ws0, outs0)
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(outs0[s], ref[s]), f"eager rerun {rep}: step {s}"


def test_graph_replays_long_rows_and_split_decode():
    """The same check on the paths the small case does not reach: rows above
    32k candidates (the chunked top-k's five launches, whose counters one launch
    clears for the next), selection given the window rows' log-sum-exp, and a
    history long enough for split decode runs merged by a second kernel
    (1,792 packed tokens: 56 history tiles plus the residual's, more than six
    per wave of an eight-wave workgroup)."""
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    B, Hkv, G, D, n, W, pool, budget, bits, R, steps = 1, 2, 2, 64, 40000, 16, 7, 1800, 2, 16, 12
    Hq = Hkv * G
    k, v = synth.random_case(41, B, Hkv, Hkv, D, n, "bf16", device="cuda")
    q_win = synth.random_tensor(42, (B, Hq, W, D), "bf16", tag="qw").cuda()
    # each window row's log-sum-exp of its causal scaled logits (float32 on the GPU)
    kk = k.float().repeat_interleave(G, dim=1).contiguous()
    lg = torch.matmul(q_win.float(), kk.transpose(-1, -2).contiguous()) / D ** 0.5
    pos = torch.arange(n, device="cuda")
    lim = n - W + torch.arange(W, device="cuda")
    lse = torch.logsumexp(lg.masked_fill(pos[None, None, None, :] > lim[None, None, :, None], float("-inf")),
                          dim=-1).contiguous()
    del kk, lg
    dec = [(synth.random_tensor(50 + s, (B, Hq, D), "bf16", tag="q").cuda(),
            synth.random_tensor(150 + s, (B, Hkv, D), "bf16", tag="kn").cuda(),
            synth.random_tensor(250 + s, (B, Hkv, D), "bf16", tag="vn").cuda()) for s in range(steps)]
    T = budget + W
    sel_ws = torch.empty(kvc.select_ws_bytes(1, B, Hq, Hkv, n, D, W, pool, budget), dtype=torch.uint8,
                         device="cuda")

    def make_cache():
        return kvc.Cache(B, Hkv, D, bits, R, q_cap=T + steps + 32, device="cuda")

    def run(cache, idx, idx_lse, dec_ws, outs):
        cache.reset()
        kvc.kvc_select_lse(q_win, k, lse, W, pool, budget, ws=sel_ws, idx=idx_lse)
        kvc.kvc_select(q_win, k, W, pool, budget, ws=sel_ws, idx=idx)
        kvc.kvc_quantize(k, v, cache, idx=idx, W=W)
        for s, (q, kn, vn) in enumerate(dec):
            kvc.kvc_decode_attn(cache, q, kn, vn, out=outs[s], ws=dec_ws)

    c0 = make_cache()
    idx0 = torch.empty(B, Hkv, budget, dtype=torch.int32, device="cuda")
    idl0 = torch.empty_like(idx0)
    ws0 = torch.zeros(kvc.decode_ws_bytes(c0, Hq), dtype=torch.uint8, device="cuda")
    outs0 = [torch.empty(B, Hq, D, dtype=torch.float32, device="cuda") for _ in range(steps)]
    run(c0, idx0, idl0, ws0, outs0)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs0]
    ref_cache = {key: t.clone() for key, t in c0.views().items()}
    ref_lse = idl0.clone()

    c1 = make_cache()
    idx1, idl1 = torch.empty_like(idx0), torch.empty_like(idx0)
    ws1 = torch.zeros_like(ws0)
    outs1 = [torch.empty_like(o) for o in outs0]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(c1, idx1, idl1, ws1, outs1)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs1:
            o.fill_(float("nan"))
        idx1.fill_(-1)
        idl1.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx0), f"replay {rep}: idx"
        assert torch.equal(idl1, ref_lse), f"replay {rep}: idx given lse"
        for s in range(steps):
            assert torch.equal(outs1[s], ref[s]), f"replay {rep}: step {s}"
        for key, t in c1.views().items():
            assert torch.equal(t, ref_cache[key]), f"replay {rep}: {key}"
        run(c0, idx0, idl0, ws0, outs0)
        torch.cuda.synchronize()
        assert torch.equal(idl0, ref_lse), f"eager rerun {rep}: idx given lse"
        for s in range(steps):
            assert torch.equal(outs0[s], ref[s]), f"eager rerun {rep}: step {s}"


def test_graph_replays_prefill_h2o_recent():
    """The fused prefill (output, accumulated attention, its variance, row
    log-sum-exp), H2O selection on it and position-only selection, captured and
    replayed: every replay equal to the eager run bit for bit."""
    gu.need_gpu()
    import kv_cache_compression_snapkv_amd as kvc

    B, Hkv, G, D, n, W, budget = 2, 2, 2, 64, 600, 16, 100
    Hq = Hkv * G
    k, v = synth.random_case(61, B, Hkv, Hkv, D, n, "bf16", device="cuda")
    q = synth.random_tensor(62, (B, Hq, n, D), "bf16", tag="q").cuda()
    pf_ws = torch.empty(kvc.prefill_ws_bytes(1, B, Hq, Hkv, n, D), dtype=torch.uint8, device="cuda")
    h_ws = torch.empty(max(kvc.h2o_ws_bytes(B, Hkv, n, W, budget), 1), dtype=torch.uint8, device="cuda")

    def buffers():
        return {"out": torch.empty(B, Hq, n, D, dtype=torch.float32, device="cuda"),
                "acc": torch.empty(B, Hkv, n, dtype=torch.float32, device="cuda"),
                "var": torch.empty(B, Hkv, dtype=torch.float32, device="cuda"),
                "lse": torch.empty(B, Hq, n, dtype=torch.float32, device="cuda"),
                "idx_h": torch.empty(B, Hkv, budget, dtype=torch.int32, device="cuda"),
                "idx_r": torch.empty(B, Hkv, budget, dtype=torch.int32, device="cuda")}

    def run(bf):
        kvc.kvc_prefill_attn(q, k, v, want_acc=True, want_var=True, ws=pf_ws, out=bf["out"], acc=bf["acc"],
                             var=bf["var"], lse=bf["lse"])
        kvc.kvc_select_h2o(bf["acc"], W, budget, ws=h_ws, idx=bf["idx_h"])
        kvc.kvc_select_recent(B, Hkv, n, W, budget, 4, idx=bf["idx_r"])

    b0 = buffers()
    run(b0)
    torch.cuda.synchronize()
    ref = {key: t.clone() for key, t in b0.items()}
    b1 = buffers()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(b1)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in b1.values():
            t.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for key, t in b1.items():
            assert torch.equal(t, ref[key]), f"replay {rep}: {key}"
        run(b0)
        torch.cuda.synchronize()
        for key, t in b0.items():
            assert torch.equal(t, ref[key]), f"eager rerun {rep}: {key}"
