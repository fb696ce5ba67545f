"""Benchmark of the compressed-KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input of the workload:
for every layer, kvc_select (window scorer + pool + top-k) and kvc_quantize
(prompt compression), then `decode_steps` decode steps, each running
kvc_decode_attn (append, flush, attention) on every layer.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--bits B]
                    [--no-cpu-baseline] [--no-sub]

Prints one JSON line.  value = decode-attention tokens/s (batch * decode steps /
time of the decode part) of the headline workload, by default the largest one:
the Llama-2-13B-shaped MHA cache with no eviction at 2 bits (40 layers x 32k
tokens x 4 sequences, 0.51 GB of packed cache per layer per step, the case bound
by HBM rather than by launch latency); the selection+quantization time per
prompt is reported beside it.  Inputs are generated on the GPU before timing
(seeded).  By default the line also carries `sub_workloads`: the same figures
for every other workload and width (the 13B shape at 4 bits, the Llama-3-8B,
Mistral pyramid and 128k long-context shapes, the 8B shape with H2O selection on
the prefill's accumulated attention, the 13B and 8B shapes at MiniKV's group size
of 16, and the 8B and 128k shapes with the window scores normalized by the
prefill's log-sum-exp), each timed the same way.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama2_13b_mha")
    ap.add_argument("--bits", type=int, default=None, help="default: 2 if the workload has it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true", help="headline workload only")
    ap.add_argument("--sub-steps", type=int, default=10, help="timed steps of each sub-workload (at most --steps)")
    ap.add_argument("--no-graph", action="store_true", help="eager launches (for counter collection)")
    ap.add_argument("--layers", type=int, default=None, help="run only the first N layers")
    ap.add_argument("--budget-policy", default="workload", choices=("workload", "var-prop", "var-inv"),
                    help="per-layer budgets: the workload's (uniform or pyramid), or proportional to the variance "
                         "of each layer's window scores or to its reciprocal (scores, budgets, then top-k)")
    ap.add_argument("--selector", default="snapkv", choices=("snapkv", "snapkv-lse", "sinks", "window", "h2o"),
                    help="prompt selection: observation-window scores (kvc_select); snapkv-lse: the same scores "
                         "given each window row's log-sum-exp from the prompt's prefill attention (kvc_prefill_attn, "
                         "run before timing as the model's prefill would), one pass over K (kvc_select_lse); "
                         "position-only with kvc_select_recent: --sinks leading tokens plus the recent window, or "
                         "the sliding window; h2o: the prefill attention of every prompt row with accumulated column "
                         "attention (kvc_prefill_attn), then heavy hitters plus the window (kvc_select_h2o)")
    ap.add_argument("--sinks", type=int, default=4)
    ap.add_argument("--streams", type=int, default=1,
                    help="prompt compression runs the layers round-robin on this many streams (they are "
                         "independent); decode stays on one stream, layer after layer")
    ap.add_argument("--flush-all", action="store_true",
                    help="MiniKV's residual policy: the prefill quantizes every complete group and the residual "
                         "is quantized whole when it reaches R")
    ap.add_argument("--group", type=int, default=32, choices=(32, 16),
                    help="quantization group: 32, or MiniKV's 16 (the decode kernel's group-16 instantiation)")
    a = ap.parse_args()
    if a.selector in ("sinks", "window") and a.budget_policy != "workload":
        ap.error("--budget-policy var-prop/var-inv needs attention scores (--selector snapkv or h2o)")
    return a


def decode_call_bytes(B, Hq, Hkv, D, bits, q_len, r_total, in_bytes, group=32):
    """Algorithmic HBM bytes of one kvc_decode_attn call (one layer)."""
    hist = q_len * D * bits // 8 * 2 + (q_len // group) * D * 4 + q_len * (D // group) * 4
    resid = r_total * D * 2 * 2
    io = B * Hq * D * in_bytes + 2 * B * Hkv * D * in_bytes + B * Hq * D * 4 + 2 * B * Hkv * D * 2
    return B * Hkv * (hist + resid) + io


DECODE_SOURCES = ("decode_kernel.h", "decode.hip", "decode_g16.hip")


def decode_src_sha256():
    """First 16 hex digits of the sha256 of the decode sources, concatenated in
    DECODE_SOURCES order (what `cat decode_kernel.h decode.hip decode_g16.hip |
    sha256sum` prints in csrc/)."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, "kv_cache_compression_snapkv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counted_traffic(workload, bits, flush_all=False, group=32):
    """HBM bytes per kvc_decode_attn call from the committed rocprofv3 counter
    summary of this workload (default residual policy; group 32, or group 16 in
    the summary named with _g16), or None when the decode sources have changed
    since the counters were taken, no summary exists, or the run uses the
    whole-residual policy."""
    import re
    if flush_all:
        return None
    tag = "" if group == 32 else f"_g{group}"
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_{bits}bit{tag}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"traffic: bytes_per_call=(\d+) workload=(\S+) bits=(\d+) decode_src_sha256=([0-9a-f]+)",
                  open(path).read())
    sha = decode_src_sha256()
    if not m or m.group(2) != workload or int(m.group(3)) != bits or m.group(4) != sha:
        return None
    return int(m.group(1))


def _spread(xs):
    """Median, 10th and 90th percentile (linear interpolation) of a list."""
    import numpy as np
    q = np.percentile(np.asarray(xs, dtype=np.float64), [50, 10, 90])
    return {"median": float(q[0]), "p10": float(q[1]), "p90": float(q[2]), "n": len(xs)}


def _timed(fn, share_s, max_reps):
    """Mean seconds per call of fn, repeated until share_s has passed (at least once)."""
    reps, t = 0, 0.0
    while reps < max_reps and (reps == 0 or t < share_s):
        t0 = time.perf_counter()
        out = fn()
        t += time.perf_counter() - t0
        reps += 1
    return t / reps, reps, out


def host_info():
    """Host cores available to this process, CPU model, BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = {i.get("internal_api", "?"): i.get("num_threads") for i in threadpool_info()}
    except Exception:  # noqa: BLE001 -- informational only
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model, "blas_threads_default": blas}


def cpu_baseline(cfg, bits, layers_budget, budget_s=12.0, group=32, flush_all=False):
    """The oracle, as it stands, on a bounded sample of the same workload: one
    (batch row, KV head) of layer 0, each stage repeated until its share of
    budget_s (selection 1/4, quantization 1/4, one decode step 1/2) is spent."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import decode as odecode
    from oracle import quant as oquant
    from oracle import select as oselect

    info = host_info()
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        # the layer is drawn where it is fastest (the GPU when there is one); only
        # the sampled (batch row, KV head) comes to the host
        p = synth.prompt_layer(cfg, 0, "cuda" if torch.cuda.is_available() else "cpu")
        qw = p["q_win"][:1, : cfg.group].float().cpu().numpy()
        kf = p["k"][:1, :1].float().cpu().numpy()
        vf = p["v"][:1, :1].float().cpu().numpy()
        del p
        n, W = cfg.prompt, cfg.window
        if cfg.budget >= 0:
            t_sel, r_sel, (idx, _) = _timed(lambda: oselect.select(qw, kf, W, cfg.pool, layers_budget[0]),
                                            budget_s / 4, 1000)
            kept = oquant.kept_positions(n, W, idx[0, 0])
        else:
            t_sel, r_sel, kept = 0.0, 0, np.arange(n)
        t_q, r_q, c = _timed(lambda: oquant.build_head_cache(kf[0, 0], vf[0, 0], kept, cfg.residual, bits, group,
                                                             flush_all=flush_all),
                             budget_s / 4, 1000)
        d = synth.decode_inputs(cfg, 0, 0, "cpu")  # small
        q = d["q"].double().numpy()[0, : cfg.group]
        kn = oquant.bf16_bits(d["k_new"].float().numpy()[0, :1])
        vn = oquant.bf16_bits(d["v_new"].float().numpy()[0, :1])
        t_dec, reps, _ = _timed(lambda: odecode.decode_step([c], q, kn, vn, cfg.residual, bits), budget_s / 2,
                                10000)
    torch.set_num_threads(os.cpu_count() or 1)
    L, B, Hkv = cfg.layers, cfg.batch, cfg.kv_heads
    step_s = t_dec * Hkv * L  # one decode step of one sequence, all layers and heads
    return {
        "value": 1.0 / step_s,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "host": info,
        "threads_used": "1 (numpy BLAS and torch limited to one thread)",
        "sample": (f"layer 0, batch row 0, KV head 0 of {cfg.name} ({cfg.group} query heads), mean per call: "
                   f"select {t_sel * 1e3:.3g} ms ({r_sel} reps), quantize {t_q * 1e3:.3g} ms ({r_q} reps), "
                   f"decode step {t_dec * 1e3:.3g} ms ({reps} reps); scaled by {Hkv} KV heads x {L} layers "
                   f"per sequence-token{' (whole-residual policy)' if flush_all else ''}"),
        "select_quantize_ms_per_prompt": (t_sel + t_q) * Hkv * L * 1e3,
    }


def run(cfg, bits, steps, warmup, graph=True, layers=None, policy="workload", selector="snapkv", sinks=4, group=32,
        streams=1, flush_all=False):
    """Time `steps` graph-replayed steps of the whole path on one workload.

    policy var-prop / var-inv: prompt compression runs kvc_window_scores for
    every layer (scores and their variance), the per-layer budgets come from
    kvc_budget_weighted on the layers' mean variances (decided once, on the host,
    from an untimed pass over the same prompts), then kvc_topk and kvc_quantize
    run per layer.  selector sinks / window: kvc_select_recent replaces
    kvc_select (first `sinks` prompt tokens plus the most recent; none for the
    sliding window).  selector h2o: kvc_prefill_attn (the causal attention of
    every prompt row and the attention each key accumulates; its variance for
    the variance policies) then kvc_select_h2o replace kvc_select; the prefill
    attention alone is also timed, for its MFMA roofline."""
    import torch

    import kv_cache_compression_snapkv_amd as kvc
    import synth

    dev = "cuda"
    print(f"[bench] {cfg.name} {bits}-bit: generating inputs", file=sys.stderr, flush=True)
    L, B, Hq, Hkv, D, n, W = cfg.layers, cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.prompt, cfg.window
    budgets, fp = kvc.kvc_budget(L, Hkv, D, n, W, cfg.decode_steps, cfg.budget, cfg.pyramid, cfg.beta,
                                 bits=bits, group=group, meta_bits=16, residual=cfg.residual)
    in_bytes = 4 if cfg.dtype == "f32" else 2
    if layers is not None:
        L = min(L, layers)
    varp = policy != "workload" and cfg.budget >= 0
    h2o = selector == "h2o" and cfg.budget >= 0
    use_lse = selector == "snapkv-lse" and cfg.budget >= 0 and not varp

    # inputs resident in HBM before timing
    prompts = [(synth.prefill_layer if h2o else synth.prompt_layer)(cfg, l, dev) for l in range(L)]
    if h2o:
        dt_code = 1 if in_bytes == 2 else 0
        accs = [torch.empty(B, Hkv, n, dtype=torch.float32, device=dev) for _ in range(L)]
        lvars = [torch.empty(B, Hkv, dtype=torch.float32, device=dev) for _ in range(L)]
        attn_out = torch.empty(B, Hq, n, D, dtype=torch.float32, device=dev)
        pf_ws = torch.empty(kvc.prefill_ws_bytes(dt_code, B, Hq, Hkv, n, D), dtype=torch.uint8, device=dev)
        if varp:
            for l in range(L):
                kvc.kvc_prefill_attn(prompts[l]["q"], prompts[l]["k"], prompts[l]["v"], want_var=True, ws=pf_ws,
                                     out=attn_out, acc=accs[l], var=lvars[l])
            score = [max(float(v.double().mean()), 1e-300) for v in lvars]
            weights = score if policy == "var-prop" else [1.0 / x for x in score]
            budgets, fp = kvc.kvc_budget_weighted(L, Hkv, D, n, W, cfg.decode_steps, cfg.budget, weights, bits=bits,
                                                  group=group, meta_bits=16, residual=cfg.residual)
        h2o_ws = torch.empty(max(kvc.h2o_ws_bytes(B, Hkv, n, W, b) for b in budgets), dtype=torch.uint8, device=dev)
    elif varp:
        N = n - W
        raws = [torch.empty(B, Hkv, N, dtype=torch.float32, device=dev) for _ in range(L)]
        lvars = [torch.empty(B, Hkv, dtype=torch.float32, device=dev) for _ in range(L)]
        sc_ws = torch.empty(max(kvc.window_scores_ws_bytes(1 if in_bytes == 2 else 0, B, Hq, Hkv, n, D, W), 1),
                            dtype=torch.uint8, device=dev)
        for l in range(L):
            kvc.kvc_window_scores(prompts[l]["q_win"], prompts[l]["k"], W, ws=sc_ws, raw=raws[l], var=lvars[l])
        score = [max(float(v.double().mean()), 1e-300) for v in lvars]
        weights = score if policy == "var-prop" else [1.0 / x for x in score]
        budgets, fp = kvc.kvc_budget_weighted(L, Hkv, D, n, W, cfg.decode_steps, cfg.budget, weights, bits=bits,
                                              group=group, meta_bits=16, residual=cfg.residual)
        tk_ws = torch.empty(max(kvc.topk_ws_bytes(B, Hkv, N, cfg.pool, b) for b in budgets), dtype=torch.uint8,
                            device=dev)
    if use_lse:
        # each window row's log-sum-exp from the prompt's prefill attention (every
        # row of the layer; its last W query rows are q_win), computed before
        # timing as the model's own prefill would
        dt_code = 1 if in_bytes == 2 else 0
        lse_out = torch.empty(B, Hq, n, D, dtype=torch.float32, device=dev)
        lse_full = torch.empty(B, Hq, n, dtype=torch.float32, device=dev)
        lse_ws = torch.empty(kvc.prefill_ws_bytes(dt_code, B, Hq, Hkv, n, D), dtype=torch.uint8, device=dev)
        lse_win = []
        for l in range(L):
            pf = synth.prefill_layer(cfg, l, dev)
            kvc.kvc_prefill_attn(pf["q"], pf["k"], pf["v"], want_acc=False, ws=lse_ws, out=lse_out, lse=lse_full)
            lse_win.append(lse_full[:, :, n - W:].contiguous())
            del pf
        del lse_out, lse_full, lse_ws
    dec = [[synth.decode_inputs(cfg, l, s, dev) for l in range(L)] for s in range(cfg.decode_steps)]
    caches, idxs = [], []
    for l in range(L):
        T = (budgets[l] + W) if cfg.budget >= 0 else n
        caches.append(kvc.Cache(B, Hkv, D, bits, cfg.residual, q_cap=T + cfg.decode_steps + 32, device=dev,
                                group=group, flush_all=flush_all))
        idxs.append(torch.empty(B, Hkv, budgets[l], dtype=torch.int32, device=dev) if cfg.budget >= 0 else None)
    sel_ws = torch.empty(max(kvc.select_ws_bytes(1 if in_bytes == 2 else 0, B, Hq, Hkv, n, D, W, cfg.pool, b)
                             for b in budgets) if cfg.budget >= 0 and not h2o else 1, dtype=torch.uint8, device=dev)
    dec_ws = torch.zeros(max(kvc.decode_ws_bytes(c, Hq, 1 if in_bytes == 2 else 0) for c in caches),
                         dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # prompt compression: the layers are independent, so they run round-robin on
    # side streams (default priority), each stream with its own workspaces
    ns = max(1, streams)
    side = [torch.cuda.Stream(device=dev) for _ in range(ns)] if ns > 1 else []
    sel_wss = [sel_ws] + [torch.empty_like(sel_ws) for _ in range(ns - 1)]
    if h2o:
        pf_wss = [pf_ws] + [torch.empty_like(pf_ws) for _ in range(ns - 1)]
        h2o_wss = [h2o_ws] + [torch.empty_like(h2o_ws) for _ in range(ns - 1)]
        attn_outs = [attn_out] + [torch.empty_like(attn_out) for _ in range(ns - 1)]
    elif varp:
        sc_wss = [sc_ws] + [torch.empty_like(sc_ws) for _ in range(ns - 1)]
        tk_wss = [tk_ws] + [torch.empty_like(tk_ws) for _ in range(ns - 1)]

    def on_streams(work):
        """work(l, k) for every layer l, on side stream k = l % ns (forked from
        and joined back to the current stream, also under graph capture)."""
        if not side:
            for l in range(L):
                work(l, 0)
            return
        cur = torch.cuda.current_stream()
        for sd in side:
            sd.wait_stream(cur)
        for l in range(L):
            with torch.cuda.stream(side[l % ns]):
                work(l, l % ns)
        for sd in side:
            cur.wait_stream(sd)

    def attn_all():
        """The prefill attention (with column sums) of every layer."""
        for l in range(L):
            p = prompts[l]
            kvc.kvc_prefill_attn(p["q"], p["k"], p["v"], ws=pf_ws, out=attn_out, acc=accs[l])

    def prefill():
        for c in caches:
            c.reset()
        if h2o:
            def h2o_one(l, k):
                p = prompts[l]
                kvc.kvc_prefill_attn(p["q"], p["k"], p["v"], ws=pf_wss[k], out=attn_outs[k], acc=accs[l])
                kvc.kvc_select_h2o(accs[l], W, budgets[l], ws=h2o_wss[k], idx=idxs[l])
                kvc.kvc_quantize(p["k"], p["v"], caches[l], idx=idxs[l], W=W)
            on_streams(h2o_one)
            return
        if varp:
            # the same layer -> stream mapping orders each layer's scores before its top-k
            on_streams(lambda l, k: kvc.kvc_window_scores(prompts[l]["q_win"], prompts[l]["k"], W, ws=sc_wss[k],
                                                          raw=raws[l], var=lvars[l]))

            def top_quant(l, k):
                kvc.kvc_topk(raws[l], cfg.pool, budgets[l], ws=tk_wss[k], idx=idxs[l])
                kvc.kvc_quantize(prompts[l]["k"], prompts[l]["v"], caches[l], idx=idxs[l], W=W)
            on_streams(top_quant)
            return

        def one(l, k):
            p = prompts[l]
            if cfg.budget >= 0 and selector in ("sinks", "window"):
                kvc.kvc_select_recent(B, Hkv, n, W, budgets[l], sinks if selector == "sinks" else 0, idx=idxs[l])
                kvc.kvc_quantize(p["k"], p["v"], caches[l], idx=idxs[l], W=W)
            elif use_lse:
                kvc.kvc_select_lse(p["q_win"], p["k"], lse_win[l], W, cfg.pool, budgets[l], ws=sel_wss[k],
                                   idx=idxs[l])
                kvc.kvc_quantize(p["k"], p["v"], caches[l], idx=idxs[l], W=W)
            elif cfg.budget >= 0:
                kvc.kvc_select(p["q_win"], p["k"], W, cfg.pool, budgets[l], ws=sel_wss[k], idx=idxs[l])
                kvc.kvc_quantize(p["k"], p["v"], caches[l], idx=idxs[l], W=W)
            else:
                kvc.kvc_quantize(p["k"], p["v"], caches[l])
        on_streams(one)

    def decode_all(nbytes=None):
        for s in range(cfg.decode_steps):
            for l in range(L):
                c, d = caches[l], dec[s][l]
                kvc.kvc_decode_attn(c, d["q"], d["k_new"], d["v_new"], out=out, ws=dec_ws)
                if nbytes is not None:
                    nbytes.append(decode_call_bytes(B, Hq, Hkv, D, bits, c.q_len, c.r_len, in_bytes, group))

    # eager pass, then capture one step into two HIP graphs (prompt compression;
    # all decode steps of all layers) so the timed replays run without host gaps
    prefill()
    call_bytes = []
    decode_all(call_bytes)
    torch.cuda.synchronize()
    if graph:
        g_pre, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pre):
            prefill()
        with torch.cuda.graph(g_dec):
            decode_all()
        torch.cuda.synchronize()
        run_pre, run_dec = g_pre.replay, g_dec.replay
    else:
        g_pre = g_dec = None
        run_pre, run_dec = prefill, decode_all
    print(f"[bench] {cfg.name} {bits}-bit: {warmup} warm-up and {steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(warmup):
        run_pre()
        run_dec()
    torch.cuda.synchronize()
    recs = []
    t_start = time.perf_counter()
    for _ in range(steps):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        run_pre()
        e1.record(stream)
        run_dec()
        e2.record(stream)
        recs.append((e0, e1, e2))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pre_ms = sum(e0.elapsed_time(e1) for e0, e1, _ in recs) / steps
    dec_ms = sum(e1.elapsed_time(e2) for _, e1, e2 in recs) / steps
    step_ms = sum(e0.elapsed_time(e2) for e0, _, e2 in recs) / steps
    ncalls = len(call_bytes)
    achieved = sum(call_bytes) / (dec_ms * 1e-3) / 1e9
    # spread over the timed steps (a graph replay is one step, so per-call times
    # are per-step means): median, p10 and p90
    call_us_steps = [e1.elapsed_time(e2) * 1e3 / ncalls for _, e1, e2 in recs]
    pre_ms_steps = [e0.elapsed_time(e1) for e0, e1, _ in recs]
    attn = None
    if h2o:
        # the prefill attention alone (every layer), for its MFMA roofline
        if graph:
            g_attn = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_attn):
                attn_all()
            run_attn = g_attn.replay
        else:
            run_attn = attn_all
        run_attn()
        torch.cuda.synchronize()
        ea = []
        for _ in range(max(1, min(steps, 5))):
            a0, a1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            a0.record(stream)
            run_attn()
            a1.record(stream)
            ea.append((a0, a1))
        torch.cuda.synchronize()
        attn_ms = sum(a0.elapsed_time(a1) for a0, a1 in ea) / len(ea)
        flops = 4.0 * D * Hq * B * n * (n + 1) / 2 * L
        peak = 2500.0 if in_bytes == 2 else 157.3
        tf = flops / (attn_ms * 1e-3) / 1e12
        attn = {"kernel": "fa_fwd_kernel + colsum_kernel (kvc_prefill_attn), every layer", "bound": "mfma",
                "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak, "traffic": None,
                "ms_per_layer": attn_ms / L, "algorithmic_flops_per_layer": flops / L,
                "flops_note": "4*D*Hq*B*n(n+1)/2 per layer: Q K^T and P V over the causal half; the column-sum pass "
                              "recomputes Q K^T and is not counted"}
        if graph:
            del g_attn
    sel = {"snapkv": "", "snapkv-lse": "window scores given the prefill's log-sum-exp (one pass over K), ",
           "sinks": f"{sinks} sinks + recent window, ", "window": "sliding window, ",
           "h2o": "H2O heavy hitters on the prefill's accumulated attention, "}[selector]
    desc = (f"{cfg.name}: {L} layers, batch {B}, {Hq} query / {Hkv} KV heads, head dim {D}, "
            f"prompt {n}, {cfg.dtype} inputs, W={W}, {sel}pool {cfg.pool}, budget "
            f"{'all' if cfg.budget < 0 else (policy + ' avg ' if varp else 'pyramid avg ' if cfg.pyramid else '') + str(cfg.budget)}, "
            f"{bits}-bit g{group} fp16 scale/zero, residual {cfg.residual}"
            f"{' (whole-residual flush)' if flush_all else ''}, {cfg.decode_steps} decode steps")
    res = {
        "desc": desc, "budgets": budgets, "footprint": fp,
        "tokens_per_s": B * cfg.decode_steps / (dec_ms * 1e-3),
        "step_ms": step_ms, "pre_ms": pre_ms, "dec_ms": dec_ms, "wall": wall, "prefill_attention": attn,
        "pre_ms_over_steps": _spread(pre_ms_steps),
        "roofline": {
            "kernel": ((f"decode_kernel<GS={group}> (+ merge_kernel"
                        + (f"; flush_kernel of {cfg.residual // group} groups on 1 step in {cfg.residual})"
                           if flush_all else f"; flush_kernel on 1 step in {group})"))
                       + ", per kvc_decode_attn call"),
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": counted_traffic(cfg.name, bits, flush_all, group),
            "avg_call_us": dec_ms * 1e3 / ncalls, "algorithmic_bytes_per_call": sum(call_bytes) / ncalls,
            "call_us_over_steps": _spread(call_us_steps),
            "traffic_note": "HBM bytes per call from rocprofv3 FETCH_SIZE/WRITE_SIZE (copy-calibrated), "
                            "profiles/decode_<workload>_<bits>bit[_g16]_hbm_counters.md; null if the decode sources changed since",
        },
    }
    del prompts, dec, caches, idxs, sel_ws, sel_wss, dec_ws, g_pre, g_dec, side
    if h2o:
        del accs, lvars, attn_out, attn_outs, pf_ws, pf_wss, h2o_ws, h2o_wss
    elif varp:
        del raws, lvars, sc_ws, tk_ws, sc_wss, tk_wss
    torch.cuda.empty_cache()
    return res


# (workload, bits, selector): every other workload and width, and the H2O path
# (workload, bits, selector, group)
SUB_WORKLOADS = (("llama2_13b_mha", 4, "snapkv", 32), ("llama2_13b_mha", 2, "snapkv", 32),
                 ("llama3_8b", 2, "snapkv", 32), ("mistral_pyramid", 2, "snapkv", 32),
                 ("long_context", 2, "snapkv", 32), ("llama3_8b", 2, "h2o", 32),
                 ("llama2_13b_mha", 2, "snapkv", 16), ("llama3_8b", 2, "snapkv", 16),
                 ("llama3_8b", 2, "snapkv-lse", 32), ("long_context", 2, "snapkv-lse", 32))


def entry(r, cfg, bits, steps, warmup, selector, group=32):
    """The figures of one workload run (a sub-workload line)."""
    e = {"workload": r["desc"], "bits": bits, "selector": selector, "group": group,
         "decode_tokens_per_s": r["tokens_per_s"],
         "avg_call_us": r["roofline"]["avg_call_us"], "ms_per_step": r["step_ms"],
         "select_quantize_ms_per_prompt": r["pre_ms"] / cfg.batch,
         "select_quantize_ms_per_prompt_over_steps": {k: (v / cfg.batch if k != "n" else v)
                                                      for k, v in r["pre_ms_over_steps"].items()},
         "steps": steps, "warmup": warmup, "roofline": r["roofline"]}
    if r["prefill_attention"] is not None:
        e["prefill_attention"] = r["prefill_attention"]
    return e


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the path shards by "
              "(batch, KV head), so each GPU would run the same kernels on its own heads)", file=sys.stderr)
        sys.exit(2)
    import synth

    cfg = synth.CONFIGS[args.workload]
    bits = args.bits or (2 if 2 in cfg.bits else cfg.bits[0])
    r = run(cfg, bits, args.steps, args.warmup, graph=not args.no_graph, layers=args.layers,
            policy=args.budget_policy, selector=args.selector, sinks=args.sinks, group=args.group,
            streams=args.streams, flush_all=args.flush_all)
    res = {
        "metric": "decode attn tokens/s + achieved HBM GB/s (% peak); select+quantize ms/prompt",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": r["desc"], "batch": cfg.batch, "prompt": cfg.prompt, "layers": cfg.layers,
                   "bits": bits, "decode_steps": cfg.decode_steps, "budget_policy": args.budget_policy,
                   "selector": args.selector, "group": args.group, "prefill_streams": args.streams,
                   "flush_all": args.flush_all},
        "select_quantize_ms_per_prompt": r["pre_ms"] / cfg.batch,
        "select_quantize_ms_per_prompt_over_steps": {k: (v / cfg.batch if k != "n" else v)
                                                     for k, v in r["pre_ms_over_steps"].items()},
        "decode_ms_per_token_all_layers": r["dec_ms"] / cfg.decode_steps,
        "decode_hbm_GBs": r["roofline"]["achieved"],
        "roofline": r["roofline"],
        "wall_s_timed": r["wall"],
        "footprint_bytes_per_prompt_token": r["footprint"]["bytes_per_prompt_token"],
    }
    if r["prefill_attention"] is not None:
        res["prefill_attention"] = r["prefill_attention"]
    if not args.no_sub:
        # every other workload and width, each timed the same way (fewer steps)
        sub_steps, sub_warm = max(1, min(args.steps, args.sub_steps)), max(1, min(args.warmup, 2))
        res["sub_workloads"] = []
        for name, sb, ssel, sg in SUB_WORKLOADS:
            if (name, sb, ssel, sg) == (args.workload, bits, args.selector, args.group):
                continue
            sc = synth.CONFIGS[name]
            h = run(sc, sb, sub_steps, sub_warm, selector=ssel, group=sg)
            res["sub_workloads"].append(entry(h, sc, sb, sub_steps, sub_warm, ssel, sg))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, bits, r["budgets"], group=args.group, flush_all=args.flush_all)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
