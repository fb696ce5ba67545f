"""ctypes binding of libkvc.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch supplies device
memory and the current stream.  Importing this module raises if the library has
not been built (there is no fallback implementation).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_F32, KVC_BF16 = 0, 1
STATUS = {0: "KVC_OK", 1: "KVC_ERR_NULL", 2: "KVC_ERR_SHAPE", 3: "KVC_ERR_DTYPE", 4: "KVC_ERR_BITS",
          5: "KVC_ERR_CAPACITY", 6: "KVC_ERR_WORKSPACE", 7: "KVC_ERR_HIP"}
EXPORTS = ("kvc_budget", "kvc_budget_weighted", "kvc_select", "kvc_select_lse", "kvc_window_scores", "kvc_topk",
           "kvc_select_recent",
           "kvc_prefill_attn", "kvc_select_h2o", "kvc_quantize", "kvc_decode_attn", "kvc_decode_attn_noalloc",
           "kvc_cache_sizes", "kvc_last_hip_error", "kvc_status_string")


class KvcError(RuntimeError):
    def __init__(self, fn, status, hip=0):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}" + (f" (hipError {hip})" if hip else ""))


class CacheStruct(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("residual", ctypes.c_int32),
                ("q_cap", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("r_cap", ctypes.c_int32), ("r_len", ctypes.c_int32), ("r_start", ctypes.c_int32),
                ("group", ctypes.c_int32), ("flush_all", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("k_meta", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p)]


class BudgetArgs(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("prompt_len", ctypes.c_int32), ("window", ctypes.c_int32), ("gen_len", ctypes.c_int32),
                ("avg_budget", ctypes.c_int32), ("pyramid", ctypes.c_int32), ("beta", ctypes.c_double),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("meta_bits", ctypes.c_int32),
                ("residual", ctypes.c_int32)]


class Footprint(ctypes.Structure):
    _fields_ = [("bits_per_element", ctypes.c_double), ("bytes_per_prompt_token", ctypes.c_double),
                ("bytes_total", ctypes.c_double), ("bytes_layout", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python kv_cache_compression_snapkv_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)
    lib.kvc_budget.argtypes = [ctypes.POINTER(BudgetArgs), ctypes.POINTER(I32), ctypes.POINTER(Footprint)]
    lib.kvc_budget_weighted.argtypes = [ctypes.POINTER(BudgetArgs), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(I32), ctypes.POINTER(Footprint)]
    lib.kvc_select.argtypes = [P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    lib.kvc_select_lse.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    lib.kvc_window_scores.argtypes = [P, P, I32, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    lib.kvc_topk.argtypes = [P, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    lib.kvc_select_recent.argtypes = [I32, I32, I32, I32, I32, I32, P, P]
    lib.kvc_prefill_attn.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P, P, SZ, P]
    lib.kvc_select_h2o.argtypes = [P, I32, I32, I32, I32, I32, P, P, SZ, P]
    lib.kvc_quantize.argtypes = [P, P, I32, I32, P, I32, I32, ctypes.POINTER(CacheStruct), P]
    lib.kvc_decode_attn.argtypes = [ctypes.POINTER(CacheStruct), P, P, P, I32, I32, P, P, SZ, P]
    lib.kvc_decode_attn_noalloc.argtypes = [ctypes.POINTER(CacheStruct), P, P, P, I32, I32, P, P]
    lib.kvc_cache_sizes.argtypes = [I32, I32, I32, I32, I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.kvc_status_string.argtypes = [I32]
    lib.kvc_status_string.restype = ctypes.c_char_p
    for f in ("kvc_budget", "kvc_budget_weighted", "kvc_select", "kvc_select_lse", "kvc_window_scores", "kvc_topk",
              "kvc_select_recent",
              "kvc_prefill_attn", "kvc_select_h2o", "kvc_quantize", "kvc_decode_attn", "kvc_decode_attn_noalloc",
              "kvc_cache_sizes", "kvc_last_hip_error"):
        getattr(lib, f).restype = I32
    return lib


lib = _load()


def _check(fn, status):
    if status != 0:
        raise KvcError(fn, status, lib.kvc_last_hip_error() if status == 7 else 0)


def _dtype(t):
    if t.dtype == torch.float32:
        return KVC_F32
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ---------------------------------------------------------------- budget
def kvc_budget(layers, kv_heads, head_dim, prompt_len, window, gen_len, avg_budget, pyramid=False,
               beta=1.0, bits=2, group=32, meta_bits=16, residual=0):
    a = BudgetArgs(layers, kv_heads, head_dim, prompt_len, window, gen_len, avg_budget, int(bool(pyramid)),
                   float(beta), bits, group, meta_bits, residual)
    out = (ctypes.c_int32 * layers)()
    fp = Footprint()
    _check("kvc_budget", lib.kvc_budget(ctypes.byref(a), out, ctypes.byref(fp)))
    return list(out), {"bits_per_element": fp.bits_per_element,
                       "bytes_per_prompt_token": fp.bytes_per_prompt_token,
                       "bytes_total": fp.bytes_total, "bytes_layout": fp.bytes_layout}


def kvc_budget_weighted(layers, kv_heads, head_dim, prompt_len, window, gen_len, avg_budget, weights, bits=2,
                        group=32, meta_bits=16, residual=0):
    """Budgets proportional to ``weights`` (one positive float per layer)."""
    if len(weights) != layers:
        raise ValueError("one weight per layer")
    a = BudgetArgs(layers, kv_heads, head_dim, prompt_len, window, gen_len, avg_budget, 0, 1.0, bits, group,
                   meta_bits, residual)
    w = (ctypes.c_double * layers)(*[float(x) for x in weights])
    out = (ctypes.c_int32 * layers)()
    fp = Footprint()
    _check("kvc_budget_weighted", lib.kvc_budget_weighted(ctypes.byref(a), w, out, ctypes.byref(fp)))
    return list(out), {"bits_per_element": fp.bits_per_element,
                       "bytes_per_prompt_token": fp.bytes_per_prompt_token,
                       "bytes_total": fp.bytes_total, "bytes_layout": fp.bytes_layout}


# ---------------------------------------------------------------- select
def window_scores_ws_bytes(dtype, B, Hq, Hkv, n, D, W):
    need = ctypes.c_size_t(0)
    _check("kvc_window_scores", lib.kvc_window_scores(None, None, dtype, B, Hq, Hkv, n, D, W, None, None, None,
                                                      ctypes.byref(need), None))
    return need.value


def kvc_window_scores(q_win, k, W, want_var=True, ws=None, raw=None, var=None, stream=None):
    """Returns raw window scores [B][Hkv][n-W] float32 (and their variance per (b, KV head))."""
    _contig(q_win, k)
    B, Hq, Wq, D = q_win.shape
    _, Hkv, n, _ = k.shape
    if Wq != W or k.dtype != q_win.dtype:
        raise ValueError("q_win must be [B][Hq][W][D] with the dtype of k")
    dt = _dtype(k)
    need = window_scores_ws_bytes(dt, B, Hq, Hkv, n, D, W)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    if raw is None:
        raw = torch.empty(B, Hkv, n - W, dtype=torch.float32, device=k.device)
    if want_var and var is None:
        var = torch.empty(B, Hkv, dtype=torch.float32, device=k.device)
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_window_scores", lib.kvc_window_scores(_ptr(q_win), _ptr(k), dt, B, Hq, Hkv, n, D, W, _ptr(raw),
                                                      _ptr(var) if want_var else None, _ptr(ws), ctypes.byref(wsb),
                                                      _stream(stream)))
    return (raw, var) if want_var else raw


def topk_ws_bytes(B, Hkv, N, pool, budget):
    need = ctypes.c_size_t(0)
    _check("kvc_topk", lib.kvc_topk(None, B, Hkv, N, pool, budget, None, None, None, ctypes.byref(need), None))
    return need.value


def kvc_topk(raw, pool, budget, want_scores=False, ws=None, idx=None, scores=None, stream=None):
    """Pool + top-k of raw scores [B][Hkv][N] float32: idx [B][Hkv][k'] (and the pooled scores)."""
    _contig(raw)
    if raw.dtype != torch.float32:
        raise TypeError("raw scores are float32")
    B, Hkv, N = raw.shape
    kk = N if budget < 0 else min(budget, N)
    need = topk_ws_bytes(B, Hkv, N, pool, budget)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=raw.device)
    if idx is None:
        idx = torch.empty(B, Hkv, kk, dtype=torch.int32, device=raw.device)
    if want_scores and scores is None:
        scores = torch.empty(B, Hkv, N, dtype=torch.float32, device=raw.device)
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_topk", lib.kvc_topk(_ptr(raw), B, Hkv, N, pool, budget, _ptr(idx),
                                    _ptr(scores) if want_scores else None, _ptr(ws), ctypes.byref(wsb),
                                    _stream(stream)))
    return (idx, scores) if want_scores else idx


def kvc_select_recent(B, Hkv, n, W, budget, sinks, idx=None, device="cuda", stream=None):
    """Sinks plus the recent window (sliding window if sinks == 0): idx [B][Hkv][k'] int32."""
    kk = (n - W) if budget < 0 else min(budget, n - W)
    if idx is None:
        idx = torch.empty(B, Hkv, max(kk, 0), dtype=torch.int32, device=device)
    elif idx.dtype != torch.int32 or tuple(idx.shape) != (B, Hkv, kk):
        raise ValueError("idx must be int32 [B][Hkv][k']")
    _contig(idx)
    _check("kvc_select_recent", lib.kvc_select_recent(B, Hkv, n, W, budget, sinks, _ptr(idx), _stream(stream)))
    return idx


def select_ws_bytes(dtype, B, Hq, Hkv, n, D, W, pool, budget):
    need = ctypes.c_size_t(0)
    _check("kvc_select", lib.kvc_select(None, None, dtype, B, Hq, Hkv, n, D, W, pool, budget, None, None,
                                        None, ctypes.byref(need), None))
    return need.value


def kvc_select(q_win, k, W, pool, budget, want_scores=False, ws=None, idx=None, scores=None, stream=None):
    """Returns idx [B][Hkv][k'] int32 (and pooled scores [B][Hkv][n-W] if asked)."""
    _contig(q_win, k)
    B, Hq, Wq, D = q_win.shape
    _, Hkv, n, _ = k.shape
    if Wq != W or k.dtype != q_win.dtype:
        raise ValueError("q_win must be [B][Hq][W][D] with the dtype of k")
    dt = _dtype(k)
    N = n - W
    kk = N if budget < 0 else min(budget, N)
    need = select_ws_bytes(dt, B, Hq, Hkv, n, D, W, pool, budget)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    if idx is None:
        idx = torch.empty(B, Hkv, kk, dtype=torch.int32, device=k.device)
    if want_scores and scores is None:
        scores = torch.empty(B, Hkv, N, dtype=torch.float32, device=k.device)
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_select", lib.kvc_select(_ptr(q_win), _ptr(k), dt, B, Hq, Hkv, n, D, W, pool, budget,
                                        _ptr(idx), _ptr(scores) if want_scores else None, _ptr(ws),
                                        ctypes.byref(wsb), _stream(stream)))
    return (idx, scores) if want_scores else idx


def kvc_select_lse(q_win, k, lse, W, pool, budget, want_scores=False, ws=None, idx=None, scores=None, stream=None):
    """kvc_select given each window row's log-sum-exp: lse float32 [B][Hq][L],
    L >= W, whose last W entries are the window rows' (kvc_prefill_attn's lse,
    L = n, or a compact [B][Hq][W]).  Same outputs as kvc_select."""
    _contig(q_win, k, lse)
    B, Hq, Wq, D = q_win.shape
    _, Hkv, n, _ = k.shape
    if Wq != W or k.dtype != q_win.dtype:
        raise ValueError("q_win must be [B][Hq][W][D] with the dtype of k")
    if lse.dtype != torch.float32 or lse.dim() != 3 or tuple(lse.shape[:2]) != (B, Hq) or lse.shape[2] < W:
        raise ValueError("lse must be float32 [B][Hq][L] with L >= W")
    dt = _dtype(k)
    N = n - W
    kk = N if budget < 0 else min(budget, N)
    need = select_ws_bytes(dt, B, Hq, Hkv, n, D, W, pool, budget)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    if idx is None:
        idx = torch.empty(B, Hkv, kk, dtype=torch.int32, device=k.device)
    if want_scores and scores is None:
        scores = torch.empty(B, Hkv, N, dtype=torch.float32, device=k.device)
    L = lse.shape[2]
    lse_w = lse.data_ptr() + (L - W) * 4  # the window rows: the last W of each row of lse
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_select_lse", lib.kvc_select_lse(_ptr(q_win), _ptr(k), ctypes.c_void_p(lse_w), L, dt, B, Hq, Hkv,
                                                n, D, W, pool, budget, _ptr(idx),
                                                _ptr(scores) if want_scores else None, _ptr(ws), ctypes.byref(wsb),
                                                _stream(stream)))
    return (idx, scores) if want_scores else idx


# ---------------------------------------------------------------- prefill
def prefill_ws_bytes(dtype, B, Hq, Hkv, n, D):
    need = ctypes.c_size_t(0)
    _check("kvc_prefill_attn", lib.kvc_prefill_attn(None, None, None, dtype, B, Hq, Hkv, n, D, None, None, None,
                                                    None, None, ctypes.byref(need), None))
    return need.value


def kvc_prefill_attn(q, k, v, want_acc=True, want_var=False, ws=None, out=None, acc=None, var=None, lse=None,
                     stream=None):
    """Causal prefill attention: out [B][Hq][n][D] float32, plus the attention
    each key accumulates, acc [B][Hkv][n] float32, and its variance [B][Hkv].
    lse (optional, float32 [B][Hq][n]) receives each row's log-sum-exp."""
    _contig(q, k, v)
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, n, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q [B][Hq][n][D], k and v [B][Hkv][n][D], one dtype")
    dt = _dtype(q)
    need = prefill_ws_bytes(dt, B, Hq, Hkv, n, D)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(B, Hq, n, D, dtype=torch.float32, device=q.device)
    if (want_acc or want_var) and acc is None:
        acc = torch.empty(B, Hkv, n, dtype=torch.float32, device=q.device)
    if want_var and var is None:
        var = torch.empty(B, Hkv, dtype=torch.float32, device=q.device)
    if lse is not None:
        _contig(lse)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, n):
            raise ValueError("lse must be float32 [B][Hq][n]")
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_prefill_attn", lib.kvc_prefill_attn(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, n, D, _ptr(out),
                                                    _ptr(acc) if (want_acc or want_var) else None,
                                                    _ptr(var) if want_var else None,
                                                    _ptr(lse) if lse is not None else None, _ptr(ws),
                                                    ctypes.byref(wsb), _stream(stream)))
    return out, (acc if (want_acc or want_var) else None), (var if want_var else None)


def h2o_ws_bytes(B, Hkv, n, W, budget):
    need = ctypes.c_size_t(0)
    _check("kvc_select_h2o", lib.kvc_select_h2o(None, B, Hkv, n, W, budget, None, None, ctypes.byref(need), None))
    return need.value


def kvc_select_h2o(acc, W, budget, ws=None, idx=None, stream=None):
    """Heavy hitters of acc [B][Hkv][n] among [0, n-W): idx [B][Hkv][k'] int32."""
    _contig(acc)
    if acc.dtype != torch.float32:
        raise TypeError("accumulated attention is float32")
    B, Hkv, n = acc.shape
    kk = (n - W) if budget < 0 else min(budget, n - W)
    need = h2o_ws_bytes(B, Hkv, n, W, budget)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=acc.device)
    if idx is None:
        idx = torch.empty(B, Hkv, max(kk, 0), dtype=torch.int32, device=acc.device)
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_select_h2o", lib.kvc_select_h2o(_ptr(acc), B, Hkv, n, W, budget, _ptr(idx), _ptr(ws), ctypes.byref(wsb),
                                                _stream(stream)))
    return idx


# ---------------------------------------------------------------- cache
class Cache:
    """One layer's compressed cache: caller-owned torch buffers + the C struct."""

    def __init__(self, batch, kv_heads, head_dim, bits, residual, q_cap, r_cap=None, device="cuda", group=32,
                 flush_all=False):
        if r_cap is None:
            r_cap = residual + group
        r_cap = 8 * ((r_cap + 7) // 8)
        q_cap = 32 * ((q_cap + 31) // 32)
        sizes = (ctypes.c_size_t * 6)()
        _check("kvc_cache_sizes", lib.kvc_cache_sizes(batch, kv_heads, head_dim, bits, group, q_cap, r_cap, sizes))
        u32 = lambda nbytes: torch.zeros(max(nbytes // 4, 1), dtype=torch.int32, device=device)
        u16 = lambda nbytes: torch.zeros(max(nbytes // 2, 1), dtype=torch.int16, device=device)
        self.k_codes, self.k_meta = u32(sizes[0]), u32(sizes[1])
        self.v_codes, self.v_meta = u32(sizes[2]), u32(sizes[3])
        self.k_res, self.v_res = u16(sizes[4]), u16(sizes[5])
        self.s = CacheStruct(batch, kv_heads, head_dim, bits, residual, q_cap, 0, r_cap, 0, 0, group, int(flush_all),
                             self.k_codes.data_ptr(), self.k_meta.data_ptr(), self.v_codes.data_ptr(),
                             self.v_meta.data_ptr(), self.k_res.data_ptr(), self.v_res.data_ptr())
        self._ws = None

    @property
    def q_len(self):
        return self.s.q_len

    @property
    def r_len(self):
        return self.s.r_len

    @property
    def r_start(self):
        return self.s.r_start

    def reset(self):
        """Mark the cache empty (buffers are kept; the next kvc_quantize refills them)."""
        self.s.q_len = 0
        self.s.r_len = 0
        self.s.r_start = 0

    def views(self):
        """Logical views of the stored state (for tests): codes/meta/residual per (b, j)."""
        s = self.s
        B, H, D, b = s.batch, s.kv_heads, s.head_dim, s.bits
        qc, rc, g = s.q_cap, s.r_cap, (s.group or 32)
        # residual ring rows, oldest first
        rows = (s.r_start + torch.arange(s.r_len, device=self.k_res.device)) % max(rc, 1)
        return {
            "k_codes": self.k_codes.view(B, H, qc, D * b // 32)[:, :, : s.q_len],
            "k_meta": self.k_meta.view(B, H, qc // g, D)[:, :, : s.q_len // g],
            "v_codes": self.v_codes.view(B, H, qc * b // 32, D)[:, :, : s.q_len * b // 32],
            "v_meta": self.v_meta.view(B, H, qc, D // g)[:, :, : s.q_len],
            "k_res": self.k_res.view(B, H, rc, D).index_select(2, rows),
            "v_res": self.v_res.view(B, H, D, rc).index_select(3, rows).transpose(-1, -2),
        }


def kvc_quantize(k, v, cache, idx=None, W=0, stream=None):
    _contig(k, v, idx)
    B, Hkv, n, D = k.shape
    k_sel = idx.shape[-1] if idx is not None else 0
    _check("kvc_quantize", lib.kvc_quantize(_ptr(k), _ptr(v), _dtype(k), n, _ptr(idx), k_sel, W,
                                            ctypes.byref(cache.s), _stream(stream)))
    return cache


def decode_ws_bytes(cache, Hq, dtype=KVC_BF16):
    """Workspace bytes of kvc_decode_attn on this cache with Hq query heads (the
    size covers every step up to the cache's capacities)."""
    need = ctypes.c_size_t(0)
    _check("kvc_decode_attn", lib.kvc_decode_attn(ctypes.byref(cache.s), None, None, None, dtype, Hq,
                                                  None, None, ctypes.byref(need), None))
    return need.value


def kvc_decode_attn(cache, q, k_new, v_new, out=None, ws=None, stream=None):
    """One decode step; returns out [B][Hq][D] float32."""
    _contig(q, k_new, v_new)
    B, Hq, D = q.shape
    if ws is None:
        need = decode_ws_bytes(cache, Hq, _dtype(q))
        if cache._ws is None or cache._ws.numel() < need:
            cache._ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
        ws = cache._ws
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    wsb = ctypes.c_size_t(ws.numel())
    _check("kvc_decode_attn", lib.kvc_decode_attn(ctypes.byref(cache.s), _ptr(q), _ptr(k_new), _ptr(v_new),
                                                  _dtype(q), Hq, _ptr(out), _ptr(ws), ctypes.byref(wsb),
                                                  _stream(stream)))
    return out


def kvc_decode_attn_noalloc(cache, q, k_new, v_new, out, stream=None):
    """kvc_decode_attn with the library's static per-device scratch instead of a
    workspace (no device allocation inside the call; `out` is the caller's)."""
    _contig(q, k_new, v_new, out)
    B, Hq, D = q.shape
    _check("kvc_decode_attn_noalloc", lib.kvc_decode_attn_noalloc(ctypes.byref(cache.s), _ptr(q), _ptr(k_new),
                                                                  _ptr(v_new), _dtype(q), Hq, _ptr(out),
                                                                  _stream(stream)))
    return out
