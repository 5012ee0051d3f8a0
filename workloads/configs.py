"""The five workload shapes of the XAttention prefill path, plus small variants.

Configs 1-5 are the shapes the library is checked and measured on.  Each one
names a generator recipe ("llm" or "video"); `get_config(i, **overrides)`
returns the same recipe at another size (fewer heads, shorter L) so the tests
can span several kernel tiles and a ragged tail at sizes the CPU oracle
finishes in seconds.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    cid: int                 # 1..5 for the named configs, 0 for ad-hoc shapes
    name: str
    recipe: str              # "llm" (RoPE'd Gaussians + shared c + sinks) or "video"
    hq: int                  # query heads
    hkv: int                 # key/value heads (GQA groups of hq // hkv)
    d: int                   # head dimension
    L: int                   # tokens
    dtype: str               # "fp32" or "bf16" (storage and input dtype)
    causal: bool
    S: int                   # antidiagonal stride
    B: int                   # sparse block size
    tau: Optional[float]     # one threshold for every head, or None -> tau_range
    tau_range: Optional[Tuple[float, float]] = None   # per-head U[lo, hi]
    seed: int = 1
    extra_sinks: int = 0     # seeded sink columns beyond positions 0..3
    rope_offset_max: int = 0  # per-query-head RoPE phase offset in U{0..max-1}
    frames: int = 0          # video recipe: frames
    frame_tokens: int = 0    # video recipe: spatial tokens per frame (h*w)
    sp_scale: float = 1.0    # video recipe: spatial-position embedding scale
    fr_scale: float = 0.5    # video recipe: per-frame embedding scale

    @property
    def nb(self) -> int:
        return self.L // self.B

    @property
    def lr(self) -> int:
        """Rows (and columns) of the stride-reshaped score matrix, L/S."""
        return self.L // self.S

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def with_(self, **kw) -> "WorkloadConfig":
        if "cid" not in kw:
            kw["cid"] = 0
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Single head, causal, fp32, L=2048, d=64, S=8, B=64, tau=0.9.
    1: WorkloadConfig(cid=1, name="single-head-fp32-2k", recipe="llm", hq=1, hkv=1,
                      d=64, L=2048, dtype="fp32", causal=True, S=8, B=64, tau=0.9,
                      seed=1, extra_sinks=0),
    # Llama-3.1-8B-shaped layer (32 q heads / 8 kv heads, d=128) at 32K, S=8.
    2: WorkloadConfig(cid=2, name="llama8b-gqa-32k", recipe="llm", hq=32, hkv=8,
                      d=128, L=32768, dtype="bf16", causal=True, S=8, B=128, tau=0.9,
                      seed=2, extra_sinks=12),
    # Same layer at 128K, S=16, tau=0.95, 32 sinks, per-head RoPE phase offsets.
    3: WorkloadConfig(cid=3, name="llama8b-gqa-128k", recipe="llm", hq=32, hkv=8,
                      d=128, L=131072, dtype="bf16", causal=True, S=16, B=128,
                      tau=0.95, seed=3, extra_sinks=28, rope_offset_max=4096),
    # Same at 256K with per-head tau ~ U[0.8, 0.95].
    4: WorkloadConfig(cid=4, name="llama8b-gqa-256k", recipe="llm", hq=32, hkv=8,
                      d=128, L=262144, dtype="bf16", causal=True, S=16, B=128,
                      tau=None, tau_range=(0.8, 0.95), seed=4, extra_sinks=28,
                      rope_offset_max=4096),
    # Video-DiT self-attention: 24 heads, L=76800 tokens in frames of 48x40 =
    # 1920 tokens (a 1920-token frame period), non-causal.  30 frames of 1920
    # tokens would be 57600 tokens, not 76800; L and the 1920-token period are
    # kept, which makes 40 frames.
    5: WorkloadConfig(cid=5, name="video-dit-76k", recipe="video", hq=24, hkv=24,
                      d=128, L=76800, dtype="bf16", causal=False, S=16, B=128,
                      tau=0.9, seed=5, frames=40, frame_tokens=1920),
}


def get_config(cid: int, **overrides) -> WorkloadConfig:
    """Config `cid`, optionally resized.  Resizing keeps the recipe and seed."""
    base = CONFIGS[cid]
    if not overrides:
        return base
    cfg = base.with_(**overrides)
    if cfg.recipe == "video" and "frames" in overrides and "L" not in overrides:
        cfg = cfg.with_(L=cfg.frames * cfg.frame_tokens)
    return cfg
