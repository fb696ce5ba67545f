"""Seeded synthetic inputs shaped like the workloads of the pages.

Shared by the tests, the benchmark and the oracle's callers; holds none of the
method's arithmetic (no scoring, selection, quantization or attention).  Every
tensor comes from a torch generator seeded by a hash of (seed, config, layer,
role, step), so any layer or decode step can be regenerated on its own, on the
CPU or on the GPU (the two devices give different but equally seeded streams;
a test always feeds both sides the same tensors).

Value recipe (no page fixes one; it is frozen here and recorded with results):
  * queries and values ~ N(0, 1);
  * keys: per-channel scale sigma_c ~ LogNormal(0, 0.5) per (layer, KV head),
    4 outlier channels x10 (the tiny case: 2 channels x8, no lognormal) --
    keys carry a few large channels (MiniKV Sec. 4.1; blog "Quantization");
  * heavy hitters: 5% of positions in [4, n-W) get gamma_h*sqrt(D)*mu, where
    mu is the unit mean of the KV group's G*W window queries; sinks 0..3 get
    gamma_s*sqrt(D)*mu (blog "Eviction": attention sinks; H2O heavy hitters);
  * model dtype: float32 (tiny case) or bfloat16 (round to nearest even).
"""

import hashlib
import math
from dataclasses import dataclass, field

import torch

GAMMA_HEAVY = 2.0
GAMMA_SINK = 4.0


@dataclass(frozen=True)
class Config:
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    prompt: int
    dtype: str            # "f32" | "bf16"
    window: int
    pool: int
    budget: int           # selected tokens per head per layer (avg); <0: keep all
    pyramid: bool
    beta: float
    bits: tuple           # quantization widths exercised
    residual: int
    decode_steps: int
    key_model: str        # "tiny" | "lognormal"
    heavy_frac: float = 0.0
    sinks: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def group(self):
        return self.q_heads // self.kv_heads


CONFIGS = {
    "tiny": Config("tiny", 1, 1, 4, 4, 64, 512, "f32", 8, 5, 64, False, 10.5, (2,),
                   16, 1, "tiny"),
    "llama3_8b": Config("llama3_8b", 32, 8, 32, 8, 128, 8192, "bf16", 32, 7, 512, False,
                        10.5, (2,), 128, 32, "lognormal", 0.05, 4),
    "mistral_pyramid": Config("mistral_pyramid", 32, 1, 32, 8, 128, 32768, "bf16", 32, 7, 128,
                              True, 10.5, (2,), 128, 64, "lognormal", 0.05, 4),
    "llama2_13b_mha": Config("llama2_13b_mha", 40, 4, 40, 40, 128, 32768, "bf16", 1, 1, -1,
                             False, 10.5, (4, 2), 128, 32, "lognormal"),
    "long_context": Config("long_context", 32, 1, 32, 8, 128, 131072, "bf16", 64, 7, 2048,
                           True, 10.5, (2,), 256, 128, "lognormal", 0.05, 4),
}


def _seed(*parts):
    h = hashlib.blake2b(repr(parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def torch_dtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def key_scales(cfg, layer, device="cpu"):
    """Per-(KV head, channel) key scale, float32 [Hkv][D]."""
    H, D = cfg.kv_heads, cfg.head_dim
    g = _gen(device, cfg.seed, cfg.name, layer, "key_scale")
    if cfg.key_model == "tiny":
        sc = torch.ones(H, D, device=device)
        ch = torch.randperm(D, generator=g, device=device)[:2]
        sc[:, ch] = 8.0
        return sc
    sc = torch.exp(0.5 * torch.randn(H, D, generator=g, device=device))
    for j in range(H):
        ch = torch.randperm(D, generator=g, device=device)[:4]
        sc[j, ch] *= 10.0
    return sc


def prompt_layer(cfg, layer, device="cpu"):
    """Prompt tensors of one layer: q_win [B][Hq][W][D], k, v [B][Hkv][n][D]."""
    B, Hq, Hkv, D, n, W = cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.prompt, cfg.window
    G = cfg.group
    f32 = torch.float32
    q_win = torch.randn(B, Hq, W, D, generator=_gen(device, cfg.seed, cfg.name, layer, "q_win"),
                        device=device, dtype=f32)
    sc = key_scales(cfg, layer, device)
    k = torch.randn(B, Hkv, n, D, generator=_gen(device, cfg.seed, cfg.name, layer, "k"),
                    device=device, dtype=f32)
    k.mul_(sc[None, :, None, :])
    v = torch.randn(B, Hkv, n, D, generator=_gen(device, cfg.seed, cfg.name, layer, "v"),
                    device=device, dtype=f32)
    if cfg.heavy_frac > 0 or cfg.sinks > 0:
        gh = _gen(device, cfg.seed, cfg.name, layer, "heavy")
        qd = q_win.to(torch_dtype(cfg)).to(f32)
        mu = qd.view(B, Hkv, G * W, D).mean(dim=2)
        mu = mu / mu.norm(dim=-1, keepdim=True)
        cand = n - W - 4
        nh = int(cfg.heavy_frac * cand)
        for b in range(B):
            for j in range(Hkv):
                if nh > 0:
                    pos = torch.randperm(cand, generator=gh, device=device)[:nh] + 4
                    k[b, j, pos] += GAMMA_HEAVY * math.sqrt(D) * mu[b, j]
                if cfg.sinks > 0:
                    k[b, j, : cfg.sinks] += GAMMA_SINK * math.sqrt(D) * mu[b, j]
    dt = torch_dtype(cfg)
    return {"q_win": q_win.to(dt), "k": k.to(dt), "v": v.to(dt)}


def prefill_layer(cfg, layer, device="cpu", n=None):
    """Prompt tensors of one layer with the queries of every prompt row:
    q [B][Hq][n][D] (its last W rows are prompt_layer's q_win), k, v
    [B][Hkv][n][D] as prompt_layer (same key model, heavy hitters and sinks).
    n < cfg.prompt takes the first n positions of a config shortened to n."""
    if n is not None and n != cfg.prompt:
        from dataclasses import replace
        cfg = replace(cfg, prompt=n, name=f"{cfg.name}@{n}")
    p = prompt_layer(cfg, layer, device)
    B, Hq, D, n, W = cfg.batch, cfg.q_heads, cfg.head_dim, cfg.prompt, cfg.window
    q_rest = torch.randn(B, Hq, n - W, D, generator=_gen(device, cfg.seed, cfg.name, layer, "q_rest"),
                         device=device, dtype=torch.float32).to(torch_dtype(cfg))
    return {"q": torch.cat([q_rest, p["q_win"]], dim=2).contiguous(), "k": p["k"], "v": p["v"]}


def decode_inputs(cfg, layer, step, device="cpu"):
    """Decode-step tensors of one layer: q [B][Hq][D], k_new, v_new [B][Hkv][D]."""
    B, Hq, Hkv, D = cfg.batch, cfg.q_heads, cfg.kv_heads, cfg.head_dim
    f32 = torch.float32
    g = _gen(device, cfg.seed, cfg.name, layer, "decode", step)
    q = torch.randn(B, Hq, D, generator=g, device=device, dtype=f32)
    k = torch.randn(B, Hkv, D, generator=g, device=device, dtype=f32)
    k.mul_(key_scales(cfg, layer, device)[None])
    v = torch.randn(B, Hkv, D, generator=g, device=device, dtype=f32)
    dt = torch_dtype(cfg)
    return {"q": q.to(dt), "k_new": k.to(dt), "v_new": v.to(dt)}


def random_case(seed, B, Hq, Hkv, D, n, dtype="bf16", device="cpu", key_scale=None):
    """Small free-form case for parity/edge tests (same value model, no planting)."""
    g = _gen(device, seed, "case", B, Hq, Hkv, D, n, dtype)
    f32 = torch.float32
    k = torch.randn(B, Hkv, n, D, generator=g, device=device, dtype=f32)
    if key_scale is not None:
        k.mul_(key_scale)
    v = torch.randn(B, Hkv, n, D, generator=g, device=device, dtype=f32)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    return k.to(dt), v.to(dt)


def random_tensor(seed, shape, dtype="bf16", device="cpu", scale=1.0, tag="t"):
    g = _gen(device, seed, tag, tuple(shape), dtype)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * scale
    return x.to(torch.float32 if dtype == "f32" else torch.bfloat16)
