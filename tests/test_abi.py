"""CPU-only checks of the C ABI: the library loads and exports every function
declared in include/kvc.h; the host-only kvc_budget equals the oracle exactly;
argument validation rejects bad calls before any device work."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

from oracle import budget as obudget

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from kv_cache_compression_snapkv_amd import _lib
    return _lib


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "kvc.h")).read()
    names = set(re.findall(r"^\s*(?:kvc_status|int|const char \*)\s*\**\s*(kvc_\w+)\s*\(", hdr, re.M))
    assert {"kvc_select", "kvc_quantize", "kvc_decode_attn", "kvc_budget"} <= names
    lib = ctypes.CDLL(_lib().LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib().EXPORTS) == names


@pytest.mark.parametrize("L,avg,pyr,beta,n,W", [
    (32, 128, True, 10.5, 32768, 32), (32, 2048, True, 10.5, 131072, 64), (32, 512, False, 1.0, 8192, 32),
    (40, 77, True, 20.0, 4096, 8), (7, 5, True, 3.0, 100, 4), (33, 1000, True, 7.25, 1500, 16),
    (1, 64, True, 10.5, 512, 8), (4, 100, True, 10.5, 120, 8), (3, -1, False, 1.0, 50, 5),
    (17, 333, True, 1.0, 100000, 1), (64, 12345, True, 123.456, 1 << 20, 100)])
def test_budget_matches_oracle_exactly(L, avg, pyr, beta, n, W):
    ks, fp = _lib().kvc_budget(L, 8, 128, n, W, 77, avg, pyr, beta, bits=2, group=32, meta_bits=16,
                               residual=128)
    assert ks == obudget.layer_budgets(L, avg, pyr, beta, n, W)
    ref = obudget.footprint(L, 8, 128, n, W, 77, avg, pyr, beta, 2, 32, 16, 128)
    for key in ref:
        assert fp[key] == pytest.approx(ref[key], rel=1e-12)


def test_budget_blog_table_digits():
    with open(os.path.join(ROOT, "tests", "golden", "blog_budget_table.json")) as f:
        g = json.load(f)
    shape = g["shape"]
    base = None
    for heads, bits, frac, b_txt, gib_txt, pct_txt in g["rows"]:
        n = shape["context"]
        avg = -1 if frac == 1.0 else int(frac * n)
        _, fp = _lib().kvc_budget(shape["layers"], heads, shape["head_dim"], n, 0, 0, avg, False, 1.0,
                                  bits=bits, group=32, meta_bits=16, residual=0)
        b = fp["bytes_per_prompt_token"]
        base = base or b
        assert f"{b:,.0f}" == b_txt and f"{b * n / 2**30:.2f}" == gib_txt and f"{b / base:.1%}" == pct_txt


def test_budget_validation():
    L = _lib()
    with pytest.raises(L.KvcError, match="SHAPE"):
        L.kvc_budget(0, 8, 128, 100, 8, 0, 10)
    with pytest.raises(L.KvcError, match="SHAPE"):
        L.kvc_budget(4, 8, 128, 100, 8, 0, 10, pyramid=True, beta=0.5)
    with pytest.raises(L.KvcError, match="BITS"):
        L.kvc_budget(4, 8, 128, 100, 8, 0, 10, bits=3)
    with pytest.raises(L.KvcError, match="BITS"):
        L.kvc_budget(4, 8, 128, 100, 8, 0, 10, group=64)


@pytest.mark.parametrize("seed", range(8))
def test_budget_weighted_matches_oracle_exactly(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 64))
    avg = int(rng.integers(0, 5000))
    n = int(rng.integers(64, 200000))
    W = int(rng.integers(1, 64))
    w = list(rng.lognormal(0.0, 1.5, L)) if seed % 2 else list(1.0 / rng.lognormal(0.0, 1.5, L))
    ks, fp = _lib().kvc_budget_weighted(L, 8, 128, n, W, 32, avg, w, bits=2, group=32, meta_bits=16, residual=128)
    assert ks == obudget.weighted_layer_budgets(w, avg, n, W)
    if all(k < n - W for k in ks):  # nothing capped
        assert sum(ks) == L * avg


def test_budget_weighted_equal_weights_is_uniform_with_same_footprint():
    L = _lib()
    ku, fu = L.kvc_budget(32, 8, 128, 8192, 32, 32, 512, bits=2, residual=128)
    kw, fw = L.kvc_budget_weighted(32, 8, 128, 8192, 32, 32, 512, [0.37] * 32, bits=2, residual=128)
    assert ku == kw and fu == fw


def test_budget_weighted_validation():
    L = _lib()
    for bad in ([1.0, 0.0], [1.0, -2.0], [1.0, float("nan")], [1.0, float("inf")]):
        with pytest.raises(L.KvcError, match="SHAPE"):
            L.kvc_budget_weighted(2, 8, 128, 100, 8, 0, 10, bad)
    with pytest.raises(L.KvcError, match="SHAPE"):
        L.kvc_budget_weighted(2, 8, 128, 100, 8, 0, -1, [1.0, 1.0])
    with pytest.raises(L.KvcError, match="SHAPE"):
        L.kvc_budget_weighted(2, 8, 128, 100, 8, 0, 10, [1e308, 1e308])  # infinite sum
    with pytest.raises(L.KvcError, match="BITS"):
        L.kvc_budget_weighted(2, 8, 128, 100, 8, 0, 10, [1.0, 1.0], bits=3)
    a = L.BudgetArgs(2, 8, 128, 100, 8, 0, 10, 0, 1.0, 2, 32, 16, 0)
    out = (ctypes.c_int32 * 2)()
    assert L.lib.kvc_budget_weighted(ctypes.byref(a), None, out, None) == 1


def test_window_scores_and_topk_validation_and_ws_query():
    L = _lib()
    need = ctypes.c_size_t(0)
    ws = L.lib.kvc_window_scores
    assert ws(None, None, 1, 2, 8, 2, 300, 128, 16, None, None, None, ctypes.byref(need), None) == 0 and need.value > 0
    assert ws(None, None, 5, 2, 8, 2, 300, 128, 16, None, None, None, ctypes.byref(need), None) == 3
    assert ws(None, None, 1, 2, 6, 4, 300, 128, 16, None, None, None, ctypes.byref(need), None) == 2
    assert ws(None, None, 1, 2, 8, 2, 300, 128, 301, None, None, None, ctypes.byref(need), None) == 2
    big = ctypes.c_size_t(1 << 24)
    P = ctypes.c_void_p(16)
    assert ws(P, P, 1, 2, 8, 2, 300, 128, 16, None, None, P, ctypes.byref(big), None) == 1  # raw NULL
    small = ctypes.c_size_t(1)
    assert ws(P, P, 1, 2, 8, 2, 300, 128, 16, P, None, P, ctypes.byref(small), None) == 6
    tk = L.lib.kvc_topk
    assert tk(None, 2, 3, 40000, 7, 100, None, None, None, ctypes.byref(need), None) == 0 and need.value > 0
    assert tk(None, 2, 3, 400, 4, 100, None, None, None, ctypes.byref(need), None) == 2   # even pool
    assert tk(None, 0, 3, 400, 5, 100, None, None, None, ctypes.byref(need), None) == 2
    assert tk(None, 2, 3, 400, 5, 100, None, None, P, ctypes.byref(big), None) == 1        # raw NULL
    assert tk(P, 2, 3, 400, 5, 100, None, None, P, ctypes.byref(big), None) == 1           # idx NULL
    assert tk(P, 2, 3, 400, 5, 0, None, None, P, ctypes.byref(small), None) == 6
    # the fused call's workspace covers both halves plus the raw scores
    assert L.select_ws_bytes(1, 2, 8, 2, 300, 128, 16, 7, 100) >= L.window_scores_ws_bytes(1, 2, 8, 2, 300, 128, 16)


def _call_select(**kw):
    L = _lib()
    args = dict(q=None, k=None, dt=1, B=1, Hq=4, Hkv=4, n=64, D=64, W=8, pool=5, budget=8)
    args.update(kw)
    need = ctypes.c_size_t(0)
    return L.lib.kvc_select(args["q"], args["k"], args["dt"], args["B"], args["Hq"], args["Hkv"], args["n"],
                            args["D"], args["W"], args["pool"], args["budget"], None, None, None,
                            ctypes.byref(need), None), need.value


def test_select_validation_and_ws_query():
    st, need = _call_select()
    assert st == 0 and need > 0
    assert _call_select(dt=7)[0] == 3
    assert _call_select(Hq=6)[0] == 2            # Hq % Hkv
    assert _call_select(D=48)[0] == 2            # D % 32
    assert _call_select(D=288)[0] == 2           # D > 256
    assert _call_select(W=0)[0] == 2
    assert _call_select(W=65)[0] == 2            # W > n
    assert _call_select(pool=4)[0] == 2          # even pool
    # with a workspace given, null inputs are rejected before any launch
    L = _lib()
    need = ctypes.c_size_t(1 << 20)
    st = L.lib.kvc_select(None, None, 1, 1, 4, 4, 64, 64, 8, 5, 8, None, None, ctypes.c_void_p(16),
                          ctypes.byref(need), None)
    assert st == 1


def test_select_lse_validation_and_ws_query():
    """kvc_select_lse: the same workspace as kvc_select; a given workspace with
    no lse, or a row stride below W, is rejected before any launch."""
    L = _lib()
    f = L.lib.kvc_select_lse
    need = ctypes.c_size_t(0)
    N = None
    assert f(N, N, N, 8, 1, 1, 4, 4, 64, 64, 8, 5, 8, N, N, N, ctypes.byref(need), N) == 0
    assert need.value == _call_select()[1]
    assert f(N, N, N, 7, 1, 1, 4, 4, 64, 64, 8, 5, 8, N, N, N, ctypes.byref(need), N) == 2   # lse stride < W
    assert f(N, N, N, 8, 1, 1, 6, 4, 64, 64, 8, 5, 8, N, N, N, ctypes.byref(need), N) == 2   # Hq % Hkv
    P = ctypes.c_void_p(16)
    big = ctypes.c_size_t(1 << 30)
    assert f(P, P, N, 8, 1, 1, 4, 4, 64, 64, 8, 5, 8, P, N, P, ctypes.byref(big), N) == 1    # no lse
    assert f(P, P, P, 8, 1, 1, 4, 4, 64, 64, 8, 5, 8, P, N, P, None, N) == 1                 # no ws_bytes


def _cache(**kw):
    L = _lib()
    c = L.CacheStruct(1, 4, 64, 2, 16, 64, 0, 48, 0, 0, 0, 0, 16, 16, 16, 16, 16, 16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_quantize_and_decode_validation():
    L = _lib()
    P = ctypes.c_void_p(16)
    q = L.lib.kvc_quantize
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(bits=3)), None) == 4
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(k_codes=None)), None) == 1
    assert q(P, P, 9, 64, None, 0, 0, ctypes.byref(_cache()), None) == 3
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(q_len=32)), None) == 5    # not empty
    assert q(P, P, 1, 200, None, 0, 0, ctypes.byref(_cache()), None) == 5           # Q > q_cap
    assert q(P, P, 1, 64, P, 100, 8, ctypes.byref(_cache()), None) == 2             # k_sel > n-W
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(r_cap=24)), None) == 5    # r_cap < R+32
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(q_cap=40)), None) == 2    # q_cap % 32
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(r_cap=52)), None) == 2    # r_cap % 8
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(r_start=4)), None) == 2   # ring start % 8
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(r_start=48)), None) == 2  # ring start >= r_cap
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(group=8)), None) == 4     # group not 16/32
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(group=16, r_cap=24)), None) == 5  # r_cap < R+16
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(group=16, q_len=16)), None) == 5  # not empty
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(q_len=16)), None) == 2    # q_len % 32
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(flush_all=2)), None) == 2  # policy not 0/1
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(flush_all=1)), None) == 2  # R=16 not a multiple of 32
    assert q(P, P, 1, 64, None, 0, 0, ctypes.byref(_cache(flush_all=1, group=16, r_len=1)), None) == 5  # not empty
    d = L.lib.kvc_decode_attn
    need = ctypes.c_size_t(0)
    assert d(ctypes.byref(_cache()), None, None, None, 1, 4, None, None, ctypes.byref(need), None) == 0
    assert need.value > 0
    small = ctypes.c_size_t(1)
    assert d(ctypes.byref(_cache()), P, P, P, 1, 4, P, P, ctypes.byref(small), None) == 6
    big = ctypes.c_size_t(need.value)
    assert d(ctypes.byref(_cache()), P, P, P, 1, 6, P, P, ctypes.byref(big), None) == 2   # Hq % Hkv
    assert d(ctypes.byref(_cache()), P, P, P, 1, 4 * 17, P, P, ctypes.byref(big), None) == 2  # G > 16
    assert d(ctypes.byref(_cache(r_len=48)), P, P, P, 1, 4, P, P, ctypes.byref(big), None) == 5
    # a flush that would overflow the packed history
    assert d(ctypes.byref(_cache(q_len=64, r_len=47)), P, P, P, 1, 4, P, P, ctypes.byref(big), None) == 5
    assert d(ctypes.byref(_cache()), P, None, P, 1, 4, P, P, ctypes.byref(big), None) == 1


def test_cache_sizes():
    L = _lib()
    out = (ctypes.c_size_t * 6)()
    bh = 6
    for g in (0, 32):
        assert L.lib.kvc_cache_sizes(2, 3, 128, 2, g, 64, 160, out) == 0
        assert list(out) == [bh * 64 * 8 * 4, bh * 2 * 128 * 4, bh * 4 * 128 * 4, bh * 64 * 4 * 4,
                             bh * 160 * 128 * 2, bh * 160 * 128 * 2]
    assert L.lib.kvc_cache_sizes(2, 3, 128, 4, 16, 64, 160, out) == 0
    assert list(out) == [bh * 64 * 16 * 4, bh * 4 * 128 * 4, bh * 8 * 128 * 4, bh * 64 * 8 * 4,
                         bh * 160 * 128 * 2, bh * 160 * 128 * 2]
    assert L.lib.kvc_cache_sizes(2, 3, 128, 3, 32, 64, 160, out) == 4
    assert L.lib.kvc_cache_sizes(2, 3, 128, 2, 8, 64, 160, out) == 4
    assert L.lib.kvc_cache_sizes(2, 3, 128, 2, 32, 65, 160, out) == 2
    assert L.lib.kvc_status_string(5).decode().startswith("cache capacity")


def test_select_recent_validation():
    """Argument checks of the position-only selector; none of these launches."""
    f = _lib().lib.kvc_select_recent
    assert f(0, 2, 100, 8, 10, 4, None, None) == 2       # B < 1
    assert f(1, 0, 100, 8, 10, 4, None, None) == 2       # Hkv < 1
    assert f(1, 2, 100, 0, 10, 4, None, None) == 2       # W < 1
    assert f(1, 2, 100, 101, 10, 4, None, None) == 2     # W > n
    assert f(1, 2, 100, 8, 10, -1, None, None) == 2      # sinks < 0
    assert f(1, 2, 100, 8, 10, 4, None, None) == 1       # idx NULL with k' > 0
    assert f(1, 2, 100, 8, 0, 4, None, None) == 0        # k' == 0: nothing to write
    assert f(1, 2, 100, 100, 10, 4, None, None) == 0     # no candidates


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; --gpus N > 1 exits non-zero with a message
    (before anything touches a GPU)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_workspace_queries_from_many_threads():
    """The workspace queries keep no state between calls: eight host threads
    querying at once get the sizes a single thread gets, for every call and
    cache shape (decode sizes do not depend on the device or the dtype)."""
    import concurrent.futures
    L = _lib()

    def dec(args):
        B, H, D, bits, R, q_cap, r_cap, G, group, dt = args
        c = L.CacheStruct(B, H, D, bits, R, q_cap, 0, r_cap, 0, 0, group, 0, 16, 16, 16, 16, 16, 16)
        need = ctypes.c_size_t(0)
        st = L.lib.kvc_decode_attn(ctypes.byref(c), None, None, None, dt, H * G, None, None, ctypes.byref(need),
                                   None)
        return st, need.value

    def sel(args):
        return L.select_ws_bytes(*args)

    dec_cases = [(B, H, D, bits, R, q_cap, r_cap, G, group, dt)
                 for (B, H, G) in ((1, 8, 4), (4, 40, 1), (8, 8, 4), (1, 1, 16))
                 for D in (64, 128, 256) for bits in (2, 4) for group in (32, 16)
                 for (R, q_cap, r_cap) in ((128, 32768, 160), (16, 64, 48), (256, 4096, 288))
                 for dt in (0, 1)]
    sel_cases = [(1, B, Hq, Hkv, n, 128, W, 7, bud) for (B, Hq, Hkv) in ((1, 32, 8), (8, 32, 8), (4, 40, 40))
                 for n in (512, 8192, 131072) for (W, bud) in ((32, 512), (64, 2048))]
    serial_dec = [dec(c) for c in dec_cases]
    serial_sel = [sel(c) for c in sel_cases]
    assert all(st == 0 and need > 0 for st, need in serial_dec)
    # the decode size is the same for both dtypes
    for i in range(0, len(dec_cases), 2):
        assert serial_dec[i] == serial_dec[i + 1]
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        for _ in range(3):
            assert list(ex.map(dec, dec_cases)) == serial_dec
            assert list(ex.map(sel, sel_cases)) == serial_sel


def test_decode_workspace_closed_form():
    """The decode workspace equals its closed form: split partials only when
    the capacity's tile count (32-token tiles, whatever the group size) exceeds
    what one workgroup per unit covers (eight waves of six tiles, four waves at
    D > 192), then units * min(64, ceil(tiles / 12)) slots of four heads' (m, l)
    and o[D].  A unit is up to four query heads of a KV head, or one head where
    the four-head kernel's LDS would exceed a CU's 160 KB (group 16 at D = 256)."""
    L = _lib()

    def need(B, H, D, R, q_cap, r_cap, G, group):
        c = L.CacheStruct(B, H, D, 2, R, q_cap, 0, r_cap, 0, 0, group, 0, 16, 16, 16, 16, 16, 16)
        n = ctypes.c_size_t(0)
        assert L.lib.kvc_decode_attn(ctypes.byref(c), None, None, None, 1, H * G, None, None, ctypes.byref(n),
                                     None) == 0
        return n.value

    def closed(B, H, D, R, q_cap, r_cap, G, group):
        nt = q_cap // 32 + (r_cap + 31) // 32
        waves = 8 if D <= 192 else 4
        if -(-nt // waves) <= 6:
            return 256
        hbs = 1 if (group == 16 and D == 256) else 4
        slots = B * H * (-(-G // hbs)) * min(64, -(-nt // 12))
        ml = -(-(slots * 4 * 8) // 256) * 256
        return max(256, ml + slots * 4 * D * 4)

    for group in (32, 16):
        for args in ((4, 40, 128, 128, 32768, 160, 1), (1, 8, 128, 256, 4096, 288, 4), (8, 8, 128, 128, 608, 160, 4),
                     (1, 1, 256, 16, 1600, 48, 16), (2, 3, 64, 16, 64, 48, 2), (1, 8, 128, 128, 8192, 160, 4),
                     (2, 2, 256, 64, 8192, 96, 4), (2, 2, 224, 64, 8192, 96, 4)):
            assert need(*args, group) == closed(*args, group), (args, group)
