"""Seeded generators for the workload configs.

Recipe "llm" (configs 1-4), per KV group g and its query heads h:
  G_q[h], G_k[g], G_v[g] ~ N(0, 1) of shape (L, d); c_g ~ N(0, 0.5^2)^d.
  Q_h = RoPE(G_q[h] + c_g, positions p - delta_h),  K_g = RoPE(G_k[g] + c_g, p).
  The shared c_g is added before RoPE, so <RoPE_i c, RoPE_j c> depends only on
  i - j: that is the local / slash structure.  RoPE uses base 10000 and the
  half-split ("rotate half") pairing, theta_k = 10000^(-2k/d).
  delta_h ~ U{0..rope_offset_max-1} per query head (0 when rope_offset_max is 0).
  Sink columns: K_g[p] += 3 * mean(Q rows of the group's query heads) for
  p in {0,1,2,3} plus `extra_sinks` distinct seeded positions in [4, L).
  V_g = G_v[g].
Recipe "video" (config 5), per head h, token t = f * frame_tokens + s:
  E_sp[h] ~ N(0,1)^(frame_tokens x d), E_fr[h] ~ N(0,1)^(frames x d),
  Q = G_q + sp_scale * E_sp[s] + fr_scale * E_fr[f], K likewise (same E),
  V ~ N(0, 1).  No RoPE, no sinks.
Per-head thresholds (config 4): tau[h] ~ U[lo, hi], rounded to float32.

Everything is computed in float64, rounded to float32, and for bf16 configs
rounded again to bfloat16 with round-to-nearest-even.  Both the HIP path and
the oracle consume the rounded tensors.  Every tensor of every head has its
own PCG64 stream keyed by (seed, stream id, index), so any subset of heads is
reproducible on its own.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .configs import WorkloadConfig

# stream ids for the per-tensor random streams
_ST_Q, _ST_K, _ST_V, _ST_C, _ST_SINK, _ST_DELTA, _ST_TAU, _ST_ESP, _ST_EFR = range(1, 10)


def _rng(seed: int, stream: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_float64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    d = x.shape[1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = pos.astype(np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[:, :half], x[:, half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=1)


@dataclass
class Workload:
    cfg: WorkloadConfig
    q_heads: List[int]       # global query-head ids held in Q (ascending)
    kv_heads: List[int]      # global kv-head ids held in K, V (ascending)
    Q: np.ndarray            # [len(q_heads)][L][d], uint16 bf16 bits or float32
    K: np.ndarray            # [len(kv_heads)][L][d]
    V: np.ndarray            # [len(kv_heads)][L][d]
    tau: np.ndarray          # float32 [hq] (all heads, always)
    sink_pos: Optional[np.ndarray] = None   # [hkv][n_sinks] (llm recipe)
    rope_offset: Optional[np.ndarray] = None  # [hq] (llm recipe)

    def q64(self, i: int) -> np.ndarray:
        return as_float64(self.Q[i], self.cfg.dtype)

    def k64(self, i: int) -> np.ndarray:
        return as_float64(self.K[i], self.cfg.dtype)

    def v64(self, i: int) -> np.ndarray:
        return as_float64(self.V[i], self.cfg.dtype)


def head_taus(cfg: WorkloadConfig) -> np.ndarray:
    if cfg.tau is not None:
        return np.full(cfg.hq, cfg.tau, dtype=np.float32)
    lo, hi = cfg.tau_range
    return _rng(cfg.seed, _ST_TAU, 0).uniform(lo, hi, size=cfg.hq).astype(np.float32)


def sink_positions(cfg: WorkloadConfig) -> np.ndarray:
    out = []
    for g in range(cfg.hkv):
        extra = np.empty(0, dtype=np.int64)
        if cfg.extra_sinks:
            extra = _rng(cfg.seed, _ST_SINK, g).choice(
                np.arange(4, cfg.L), size=cfg.extra_sinks, replace=False)
        out.append(np.sort(np.concatenate([np.arange(min(4, cfg.L)), extra])))
    return np.stack(out).astype(np.int64)


def rope_offsets(cfg: WorkloadConfig) -> np.ndarray:
    if cfg.rope_offset_max <= 0:
        return np.zeros(cfg.hq, dtype=np.int64)
    return _rng(cfg.seed, _ST_DELTA, 0).integers(0, cfg.rope_offset_max, size=cfg.hq)


def _llm_group(cfg: WorkloadConfig, g: int, sinks: np.ndarray, offs: np.ndarray):
    L, d = cfg.L, cfg.d
    c = _rng(cfg.seed, _ST_C, g).normal(0.0, 0.5, size=d)
    pos = np.arange(L, dtype=np.int64)
    qs = []
    for h in range(g * cfg.group, (g + 1) * cfg.group):
        gq = _rng(cfg.seed, _ST_Q, h).standard_normal((L, d))
        qs.append(_rope(gq + c, pos - offs[h]))
    qmean = np.mean([q.mean(axis=0) for q in qs], axis=0)
    gk = _rng(cfg.seed, _ST_K, g).standard_normal((L, d))
    k = _rope(gk + c, pos)
    k[sinks[g]] += 3.0 * qmean
    v = _rng(cfg.seed, _ST_V, g).standard_normal((L, d))
    return ([_store(q, cfg.dtype) for q in qs], _store(k, cfg.dtype), _store(v, cfg.dtype))


def _video_head(cfg: WorkloadConfig, h: int):
    L, d, ft = cfg.L, cfg.d, cfg.frame_tokens
    t = np.arange(L)
    s_of, f_of = t % ft, t // ft
    esp = _rng(cfg.seed, _ST_ESP, h).standard_normal((ft, d))
    efr = _rng(cfg.seed, _ST_EFR, h).standard_normal((cfg.frames, d))
    emb = cfg.sp_scale * esp[s_of] + cfg.fr_scale * efr[f_of]
    q = _rng(cfg.seed, _ST_Q, h).standard_normal((L, d)) + emb
    k = _rng(cfg.seed, _ST_K, h).standard_normal((L, d)) + emb
    v = _rng(cfg.seed, _ST_V, h).standard_normal((L, d))
    return ([_store(q, cfg.dtype)], _store(k, cfg.dtype), _store(v, cfg.dtype))


def generate(cfg: WorkloadConfig, kv_heads: Optional[Sequence[int]] = None,
             threads: Optional[int] = None) -> Workload:
    """Inputs of `cfg` for the given KV heads (default: all) and their query heads."""
    if cfg.L % cfg.B or cfg.B % cfg.S or cfg.hq % cfg.hkv:
        raise ValueError("config shape must satisfy L % B == 0, B % S == 0, hq % hkv == 0")
    if cfg.recipe == "video" and cfg.frames * cfg.frame_tokens != cfg.L:
        raise ValueError("video recipe needs L == frames * frame_tokens")
    kvs = list(range(cfg.hkv)) if kv_heads is None else sorted(set(int(g) for g in kv_heads))
    sinks = sink_positions(cfg) if cfg.recipe == "llm" else None
    offs = rope_offsets(cfg) if cfg.recipe == "llm" else None
    if threads is None:
        threads = max(1, min(len(kvs), len(os.sched_getaffinity(0)), 16))

    def one(g):
        if cfg.recipe == "llm":
            return _llm_group(cfg, g, sinks, offs)
        return _video_head(cfg, g)

    if threads > 1 and len(kvs) > 1:
        with cf.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(one, kvs))
    else:
        parts = [one(g) for g in kvs]
    Q = np.stack([q for p in parts for q in p[0]])
    K = np.stack([p[1] for p in parts])
    V = np.stack([p[2] for p in parts])
    qh = [h for g in kvs for h in range(g * cfg.group, (g + 1) * cfg.group)]
    return Workload(cfg=cfg, q_heads=qh, kv_heads=kvs, Q=Q, K=K, V=V, tau=head_taus(cfg),
                    sink_pos=sinks, rope_offset=offs)
