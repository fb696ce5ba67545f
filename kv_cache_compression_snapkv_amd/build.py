"""Build libkvc.so (all HIP kernels + the C ABI) in-tree for gfx950.

    python kv_cache_compression_snapkv_amd/build.py   (or __graft_entry__.build())

Each source is compiled to an object in parallel, then linked.  Flags:
  --offload-arch=gfx950                      MI355X only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed fp32 instructions
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division (quantizer scale)
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvc.so")
SOURCES = ["budget.cpp", "quantize.hip", "decode.hip", "decode_g16.hip", "select.hip", "prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-result",
]


# Per-source extras.  Every source's values are never NaN for finite inputs
# (decode, selection and prefill: logits, softmax weights, -inf masks;
# quantization: group extremes, and codes whose groups have a zero or infinite
# scale use a zero-point of 0), so fmin/fmax need no canonicalization and the
# DPP lane exchanges fold into v_min/v_max_f32_dpp.
_NO_NANS = ["-fno-honor-nans"]
EXTRA = {"decode.hip": _NO_NANS, "decode_g16.hip": _NO_NANS, "select.hip": _NO_NANS, "prefill.hip": _NO_NANS,
         "quantize.hip": _NO_NANS}


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
