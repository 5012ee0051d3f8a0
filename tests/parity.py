"""Helpers shared by the GPU parity tests: device upload of seeded inputs and
the comparison rules.

Tolerances:
  scores   |gpu - oracle| <= 1e-3 * |oracle| + 1e-12 for every entry.
  masks    bit-exact on every row whose oracle prefix sum at the cut is not
           within 1e-4 of tau.  A row inside that band (tau band) may move
           the cut by one block either way, but its GPU set must still be a
           top set of the oracle's ranking: k*-1, k* or k*+1 blocks, no
           unselected block scoring more than TIE_REL (relative) above a
           selected one (fp32 scoring can swap such near-ties, and inside
           the band either side of the cut is a correct reading of the
           >= tau rule at the oracle's own precision).  Outside the tau band
           a row whose two oracle scores at the cut lie within TIE_REL of
           each other (tie band) gets no exemption: any mismatch fails, with
           the tie status named in the message.  Both band counts are
           reported.
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
    tau_band: int = 0        # rows inside the tau band (equal or not)
    tau_band_moved: int = 0  # of which the GPU set differs (a top set, see is_top_set)
    tie_band: int = 0        # rows whose two scores at the cut are a near-tie
    failures: List[str] = field(default_factory=list)

    def summary(self) -> str:
        return (f"rows {self.rows} equal {self.equal} tau-band {self.tau_band} "
                f"(differing {self.tau_band_moved}) tie-band {self.tie_band} "
                f"failures {len(self.failures)}")


def in_tau_band(sel: O.Selection, tau: float) -> bool:
    """The oracle's prefix sum at the cut (P_k* or P_k*-1) lies within
    TAU_BAND of tau."""
    k = sel.kstar
    return min(abs(sel.prefix(k) - tau), abs(tau - sel.prefix(k - 1))) <= TAU_BAND


def in_tie_band(sorted_scores: np.ndarray, sel: O.Selection) -> bool:
    """The last selected and the first unselected oracle scores are within
    TIE_REL of each other (fp32 scoring error could swap them)."""
    k = sel.kstar
    return bool(k < sel.n_valid and
                (sorted_scores[k - 1] - sorted_scores[k]) <= TIE_REL * sorted_scores[k - 1])


def is_top_set(sel: O.Selection, sorted_scores: np.ndarray, gset: List[int]) -> bool:
    """gset has k*-1, k* or k*+1 valid blocks and is a top set of the
    oracle's scores up to near-ties: no unselected valid block scores more
    than TIE_REL above the lowest selected one."""
    n = sel.n_valid
    if not (sel.kstar - 1 <= len(gset) <= sel.kstar + 1) or not gset:
        return False
    if len(set(gset)) != len(gset) or min(gset) < 0 or max(gset) >= n:
        return False
    by_kb = np.empty(n, dtype=np.float64)
    by_kb[np.asarray(sel.order)] = np.asarray(sorted_scores, dtype=np.float64)
    inside = np.zeros(n, dtype=bool)
    inside[gset] = True
    if inside.all():
        return True
    return bool(by_kb[~inside].max() <= by_kb[inside].min() * (1.0 + TIE_REL))


def classify_rows(sels: Sequence[O.Selection], sorted_scores: Sequence[np.ndarray],
                  gpu_sets: Sequence[List[int]], taus: Sequence[float],
                  labels: Sequence[str]) -> MaskReport:
    """Compare GPU selections with the oracle's, row by row (strict rule:
    outside the tau band only identical sets pass)."""
    rep = MaskReport()
    for sel, srt, gset, tau, lab in zip(sels, sorted_scores, gpu_sets, taus, labels):
        rep.rows += 1
        k = sel.kstar
        tau_b = in_tau_band(sel, tau)
        tie_b = in_tie_band(srt, sel)
        rep.tau_band += tau_b
        rep.tie_band += tie_b
        gset = [int(x) for x in gset]
        if [int(x) for x in sel.selected] == gset:
            rep.equal += 1
            continue
        if tau_b and is_top_set(sel, srt, gset):
            rep.tau_band_moved += 1
            continue
        rep.failures.append(
            f"{lab}: oracle k*={k} {[int(x) for x in sel.selected][:12]}... gpu k={len(gset)} "
            f"{gset[:12]}... (tau band {tau_b}, tie band {tie_b}, P_k*={sel.prefix(k)!r}, "
            f"P_k*-1={sel.prefix(k - 1)!r}, tau={tau!r})")
    return rep
