"""Helpers shared by the GPU parity tests: device upload of seeded inputs and
the comparison rules.

Tolerances:
  scores   |gpu - oracle| <= 1e-3 * |oracle| + 1e-12 for every entry.
  masks    bit-exact; a row may differ only if the oracle's prefix sum at the
           cut is within 1e-4 of tau (tau band) or its two scores at the cut
           are within TIE_REL of each other (tie band: fp32 scoring error can
           swap them).  Both counts are reported.
  outputs  bf16: max |diff| <= 2e-2 and ||diff||_2 / ||oracle||_2 <= 5e-3;
           fp32: max |diff| <= 1e-4.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence

import numpy as np

import oracle as O

TAU_BAND = 1e-4
TIE_REL = 1e-4
SCORE_RTOL = 1e-3
SCORE_ATOL = 1e-12


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda")


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_scores_close(gpu: np.ndarray, ora: np.ndarray, what: str = "scores") -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ora)
    bound = SCORE_RTOL * np.abs(ora) + SCORE_ATOL
    bad = err > bound
    rel = float(np.max(err / (np.abs(ora) + 1e-30))) if ora.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries beyond tolerance; worst at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)} "
                           f"gpu={gpu.flat[np.argmax(err - bound)]!r} "
                           f"oracle={ora.flat[np.argmax(err - bound)]!r}")
    return rel


def assert_outputs_close(gpu: np.ndarray, ora: np.ndarray, dtype: str, what: str = "O") -> Dict:
    diff = np.abs(gpu - ora)
    mx = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(gpu - ora) / max(np.linalg.norm(ora), 1e-300))
    if dtype == "bf16":
        assert mx <= 2e-2 and rel <= 5e-3, f"{what}: max-abs {mx:.3e}, rel-L2 {rel:.3e}"
    else:
        assert mx <= 1e-4, f"{what}: max-abs {mx:.3e}"
    return {"max_abs": mx, "rel_l2": rel}


def gpu_selected(idx_row: np.ndarray, count: int) -> List[int]:
    return [int(v) for v in idx_row[:count]]


def mask_bits(words: np.ndarray, NB: int) -> List[int]:
    out = []
    for kb in range(NB):
        if (int(words[kb // 64]) >> (kb % 64)) & 1:
            out.append(kb)
    return out


@dataclass
class MaskReport:
    rows: int = 0
    equal: int = 0
    tau_band: int = 0
    tie_band: int = 0
    failures: List[str] = field(default_factory=list)


def classify_rows(sels: Sequence[O.Selection], sorted_scores: Sequence[np.ndarray],
                  gpu_sets: Sequence[List[int]], taus: Sequence[float],
                  labels: Sequence[str]) -> MaskReport:
    """Compare GPU selections with the oracle's, row by row."""
    rep = MaskReport()
    for sel, srt, gset, tau, lab in zip(sels, sorted_scores, gpu_sets, taus, labels):
        rep.rows += 1
        if list(sel.selected) == list(gset):
            rep.equal += 1
            continue
        k = sel.kstar
        near_tau = min(abs(sel.prefix(k) - tau), abs(tau - sel.prefix(k - 1))) <= TAU_BAND
        if near_tau:
            rep.tau_band += 1
            continue
        if k < sel.n_valid and (srt[k - 1] - srt[k]) <= TIE_REL * srt[k - 1]:
            rep.tie_band += 1
            continue
        rep.failures.append(f"{lab}: oracle k*={k} {list(sel.selected)[:12]}... gpu "
                            f"k={len(gset)} {list(gset)[:12]}...")
    return rep
