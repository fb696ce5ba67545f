"""Compressed-KV-cache hot path for AMD MI355X (gfx950).

SnapKV/PyramidKV window selection -> KIVI/MiniKV 2/4-bit group quantization ->
single-query decode attention over the packed cache plus a bf16 residual, all in
hand-written HIP kernels behind the C ABI of ``include/kvc.h``.  This package is
the thin Python binding (same entry-point names); it needs ``libkvc.so``, built
by ``python kv_cache_compression_snapkv_amd/build.py`` (or ``__graft_entry__.build()``).
"""

from ._lib import (Cache, KvcError, LIB_PATH, decode_ws_bytes, h2o_ws_bytes, kvc_budget,  # noqa: F401
                   kvc_budget_weighted, kvc_decode_attn, kvc_decode_attn_noalloc, kvc_prefill_attn, kvc_quantize,
                   kvc_select, kvc_select_h2o, kvc_select_lse,
                   kvc_select_recent, kvc_topk, kvc_window_scores, prefill_ws_bytes, select_ws_bytes, topk_ws_bytes,
                   window_scores_ws_bytes)
