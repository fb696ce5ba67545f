"""CPU oracle for the compressed-KV-cache path: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports it, and this
package never imports the product path: the two share no code, no tables and no
constants.  The seeded input generators live in ``synth`` and hold none of the
method's arithmetic.

Sources (cited by page title and section in each function):
  * "KV Cache Compression: Eviction and Quantization" (blog): the budget
    script and table, the eviction rules (sliding window, attention sinks), the
    ``round_to`` quantizer, the ``attention()`` hook.
  * "PyramidKV: Dynamic KV Cache Compression based on Pyramidal Information
    Funneling": budget allocation and SnapKV-style selection.
  * "MiniKV: Pushing the Limits of LLM Inference via 2-Bit Layer-Discriminative
    KV Cache": problem statement (Eq. 1, Def. 2.1), the pyramid and variance
    policies (Sec. 4.2), the INT2 kernels and streaming residual (Sec. 4.4),
    Algorithm 1, the group size of Sec. 5.1, the KV-size analysis.
  * "CSKV: Training-Efficient Channel Shrinking for KV Cache in Long-Context
    Scenarios": the footprint claim of the introduction.
  * MiniKV Sec. 4.3 "Selective KV Compatible Attention Kernels" (Fig. 9): the
    prefill attention that also returns the attention each key accumulates;
    blog "Eviction" and PyramidKV "Baselines": H2O heavy hitters.

Precision: scores and attention in float64; the quantizer in exact IEEE float32
with float16 scale/zero (numpy float32 ops and float16 casts round to nearest
even); bfloat16 by round-to-nearest-even bit arithmetic.

Parity status of each function (pins live in ``tests/test_oracle_*.py``):
  budget.*            pinned (blog table, MiniKV example, CSKV/PyramidKV claims,
                      pyramid invariants, weighted-budget closed forms)
  select.*            pinned (torch softmax/max_pool1d, brute force, invariants,
                      variance closed forms; recent_select: the blog's sink/window
                      configurations, PyramidKV's split, a top-k route)
  quant.*             pinned (error bound, exact-nearest brute force, integer
                      groups, blog round_to, pack round trip; group 16: layout
                      through packing, integer groups, residual closed forms)
  decode.*            pinned (torch SDPA, dense special case, convex hull, blog
                      attention hook semantics, incremental flush == batch, at
                      groups 32 and 16)
  prefill.*           pinned (torch SDPA for the output, pure-Python brute force
                      and the harmonic closed form for the column sums, the
                      row-mass invariant, the last W rows == window scores,
                      H2O selection by brute-force sort, variance closed forms;
                      row_lse: brute force, max/log bounds, equal-keys closed form)
"""

from . import budget, select, quant, decode, prefill  # noqa: F401
