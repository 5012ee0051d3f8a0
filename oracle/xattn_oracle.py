"""Plain float64 CPU oracle of the XAttention prefill path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the library never does, and it
shares no code with the HIP kernels.  Everything here is numpy float64 on the
exact input values, written to be checked against the pages by eye.

Source: "XAttention: Block Sparse Attention with Antidiagonal Scoring"
(papercache.org summary, section 2.2 "Threshold Block Selection": the
find_blocks equation and Algorithm 1; the chapterpal.com page, Knowl 2, restates
both in English).  The block-sparse attention step follows section 1 (step 3,
"Block Sparse Attention") of the same summary and step 4 of the dtcms.com
worked example (softmax over the selected entries at 1/sqrt(d)).

Readings where the pages are silent (each is pinned by a test):
  * "append" in Algorithm 1 concatenates along the feature axis, so a reshaped
    query row pairs query sub-row a with key sub-row S-1-a: the product entry
    is the sum of the S-th antidiagonal of one SxS tile of Q K^T.
  * causal: reshaped column c is masked when c > R (reshaped row).  The
    diagonal entry c == R keeps its whole antidiagonal.
  * block mass = sum of A_approx over the (B/S)x(B/S) tile, divided by B/S so
    every query-block row sums to 1 (tau lies in (0, 1]).
  * find_blocks runs per (head, query block) over the valid key blocks
    (kb <= qb when causal), in order of mass descending, lower kb first on
    ties; the cut is the first prefix whose mass is >= tau; tau >= 1 (or a
    tau never reached because of rounding) selects every valid block.
  * sparse attention: softmax at 1/sqrt(d) renormalised over the keys of the
    selected blocks (and j <= i when causal); a row with no key outputs 0.
  * sampling patterns other than the antidiagonal (named, not defined, in the
    pattern ablation): diagonal = key sub-row a for query sub-row a; random =
    a seeded permutation of the key sub-rows, drawn by the caller.
  * the video warm-up: denoising steps count from 0; steps < warmup (5) run
    dense attention, the rest the sparse path.
  * threshold prediction: each head takes k = 0 .. R reduction steps (x0.9
    each) and exactly M steps are distributed; the garbled recurrence is read
    as the 0/1 (R = 1) or multiple-choice selection DP; the performance proxy
    is minus the summed relative squared output error (parity unpinned against
    the pages' accuracy numbers, which need a trained model).
  * Top-K / Top-Ratio (the ablation's alternative cut rules, named but not
    defined on the pages): the same ranking as find_blocks, cut at a fixed
    count -- k blocks (K tokens / B), or the nearest integer to ratio * |valid|
    -- clamped to [1, |valid|].
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# Step 1 -- strided antidiagonal sums (section 2.1 / 2.2; Algorithm 1's
# reshape-and-multiply).  A[R, c] is the sum of the elements (i, j) of Q K^T
# inside the SxS tile (R, c) that lie on its antidiagonal i + j = (R+c)S + S-1.
# ---------------------------------------------------------------------------
def antidiagonal_sums(Q: np.ndarray, K: np.ndarray, S: int,
                      rows: Optional[range] = None) -> np.ndarray:
    """A[R, c] = sum_{a<S} <Q[R*S + a], K[c*S + S-1-a]> for R in `rows`, all c.

    Q: float64 (Lq, d), K: float64 (Lk, d) (the path uses Lq == Lk == L).  Written as the explicit tile-antidiagonal sum: the
    query rows with phase a against the key rows with phase S-1-a.
    """
    rows = range(Q.shape[0] // S) if rows is None else rows
    r0, r1 = rows.start, rows.stop
    Lk = K.shape[0] // S
    A = np.zeros((r1 - r0, Lk), dtype=np.float64)
    for a in range(S):
        q_phase = Q[r0 * S + a: r1 * S: S]          # rows R*S + a
        k_phase = K[S - 1 - a: Lk * S: S]           # rows c*S + S-1-a
        A += q_phase @ k_phase.T
    return A


def pattern_sums(Q: np.ndarray, K: np.ndarray, S: int, phase: Sequence[int],
                 rows: Optional[range] = None) -> np.ndarray:
    """A[R, c] = sum_{a<S} <Q[R*S + a], K[c*S + phase[a]]>: the SxS tile of
    Q K^T sampled at one entry per query sub-row a, the key sub-row given by
    the permutation `phase`.  Sampling patterns of the ablation on pattern
    geometry (chapterpal.com Knowl 9, "Pattern Geometry": antidiagonal,
    diagonal and random sampling at the same stride; papercache.org summary,
    ablation on the antidiagonal pattern): phase[a] = S-1-a is the antidiagonal
    of antidiagonal_sums, phase[a] = a the main diagonal, a seeded random
    permutation the random pattern (one sample per query and key sub-row)."""
    phase = [int(x) for x in phase]
    assert sorted(phase) == list(range(S)), "phase must be a permutation of 0..S-1"
    rows = range(Q.shape[0] // S) if rows is None else rows
    r0, r1 = rows.start, rows.stop
    Lk = K.shape[0] // S
    A = np.zeros((r1 - r0, Lk), dtype=np.float64)
    for a in range(S):
        A += Q[r0 * S + a: r1 * S: S] @ K[phase[a]: Lk * S: S].T
    return A


# ---------------------------------------------------------------------------
# Step 2 -- A_approx = Softmax(A / sqrt(d_h * S)) per reshaped row (Algorithm 1),
# with the causal reading c > R masked.
# ---------------------------------------------------------------------------
def approx_attention(A: np.ndarray, d: int, S: int, causal: bool, row0: int) -> np.ndarray:
    Z = A / math.sqrt(d * S)
    if causal:
        R = np.arange(row0, row0 + A.shape[0])[:, None]
        c = np.arange(A.shape[1])[None, :]
        Z = np.where(c > R, -np.inf, Z)
    m = Z.max(axis=1, keepdims=True)
    E = np.exp(Z - m)
    return E / E.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Step 3 -- block mass: sum of A_approx over each (B/S)x(B/S) tile, / (B/S).
# ---------------------------------------------------------------------------
def block_mass(P: np.ndarray, B: int, S: int) -> np.ndarray:
    """P: rows of whole query blocks (a multiple of B/S rows), L/S columns."""
    bs = B // S
    nq = P.shape[0] // bs
    nk = P.shape[1] // bs
    tiles = P[: nq * bs, : nk * bs].reshape(nq, bs, nk, bs)
    return tiles.sum(axis=(1, 3)) / bs


def block_scores(Q: np.ndarray, K: np.ndarray, S: int, B: int, causal: bool,
                 qblocks: Optional[Sequence[int]] = None, chunk: int = 64,
                 phase: Optional[Sequence[int]] = None) -> np.ndarray:
    """Block scores [len(qblocks)][NB] of one head (Q: its queries, K: its group's keys).

    Follows Algorithm 1 per query block b: reshaped product, scaled softmax,
    then the tile sums that find_blocks takes.  Causal entries kb > qb are 0.
    Consecutive query blocks are evaluated `chunk` at a time (their rows do
    not interact).  `phase` (default: the antidiagonal) selects another
    sampling pattern through pattern_sums; the rest is unchanged.
    """
    L, d = Q.shape
    NB = L // B
    bs = B // S
    qblocks = list(range(NB)) if qblocks is None else [int(b) for b in qblocks]
    out = np.zeros((len(qblocks), NB), dtype=np.float64)
    i = 0
    while i < len(qblocks):
        j = i + 1
        while j < len(qblocks) and j - i < chunk and qblocks[j] == qblocks[j - 1] + 1:
            j += 1
        b0, b1 = qblocks[i], qblocks[j - 1] + 1
        rr = range(b0 * bs, b1 * bs)
        A = antidiagonal_sums(Q, K, S, rr) if phase is None else pattern_sums(Q, K, S, phase, rr)
        P = approx_attention(A, d, S, causal, b0 * bs)
        out[i:j] = block_mass(P, B, S)
        i = j
    return out


# ---------------------------------------------------------------------------
# Step 4 -- find_blocks(A, tau) = argmin_{blocks} |blocks| s.t. mass >= tau.
# The smallest set reaching tau is a prefix of the blocks sorted by mass.
# ---------------------------------------------------------------------------
@dataclass
class Selection:
    selected: np.ndarray     # ascending key-block ids
    kstar: int               # number selected
    order: np.ndarray        # valid key blocks, mass descending, lower kb first on ties
    csum: np.ndarray         # inclusive prefix sums of mass in `order` (float64)
    n_valid: int

    def prefix(self, k: int) -> float:
        """P_k (P_0 = 0)."""
        return 0.0 if k <= 0 else float(self.csum[k - 1])


def find_blocks(mass_row: np.ndarray, n_valid: int, tau: float) -> Selection:
    mass = np.asarray(mass_row, dtype=np.float64)[:n_valid]
    kb = np.arange(n_valid)
    order = np.lexsort((kb, -mass))          # primary: mass desc; secondary: kb asc
    csum = np.cumsum(mass[order])            # sequential float64 accumulation
    if tau >= 1.0:
        k = n_valid
    else:
        hit = np.nonzero(csum >= tau)[0]
        k = int(hit[0]) + 1 if hit.size else n_valid
    sel = np.sort(order[:k])
    return Selection(selected=sel, kstar=k, order=order, csum=csum, n_valid=n_valid)


def _ranked_prefix(mass_row: np.ndarray, n_valid: int, k: int) -> Selection:
    """The first k valid blocks in the ranking of find_blocks (score
    descending, lower block first on equal scores)."""
    mass = np.asarray(mass_row, dtype=np.float64)[:n_valid]
    kb = np.arange(n_valid)
    order = np.lexsort((kb, -mass))
    csum = np.cumsum(mass[order])
    k = max(1, min(int(k), n_valid))
    return Selection(selected=np.sort(order[:k]), kstar=k, order=order, csum=csum,
                     n_valid=n_valid)


def find_blocks_topk(mass_row: np.ndarray, n_valid: int, k_blocks: int) -> Selection:
    """Top-K selection of the ablation on block selection strategies
    (chapterpal.com Knowl 9, "Selection Strategy"; papercache.org summary,
    ablation "block selection strategy"): a fixed number of key blocks per
    query block, the k highest-scoring valid ones.  The pages give K in tokens
    (8192); here k counts blocks (K / B).  A row with fewer valid blocks keeps
    all of them; k >= 1."""
    return _ranked_prefix(mass_row, n_valid, k_blocks)


def topratio_count(n_valid: int, ratio: float) -> int:
    """Blocks kept by Top-Ratio: the nearest integer to ratio * n_valid (halves
    round up), at least 1 and at most n_valid.  Evaluated in float64 from the
    float32 ratio, as floor(r * n + 0.5)."""
    r = float(np.float32(ratio))
    return max(1, min(n_valid, int(math.floor(r * n_valid + 0.5))))


def find_blocks_topratio(mass_row: np.ndarray, n_valid: int, ratio: float) -> Selection:
    """Top-Ratio selection of the same ablation (ratio 27% on the pages): the
    highest-scoring topratio_count(n_valid, ratio) valid blocks of the row."""
    return _ranked_prefix(mass_row, n_valid, topratio_count(n_valid, ratio))


def select_all(scores: np.ndarray, causal: bool, tau: float,
               qblocks: Optional[Sequence[int]] = None) -> List[Selection]:
    """find_blocks for every row of `scores` (rows are query blocks `qblocks`)."""
    NB = scores.shape[1]
    qblocks = list(range(scores.shape[0])) if qblocks is None else list(qblocks)
    return [find_blocks(scores[i], (qb + 1) if causal else NB, tau)
            for i, qb in enumerate(qblocks)]


def to_mask(sel: Selection, NB: int) -> np.ndarray:
    """Bitmask words (uint64, bit kb % 64 of word kb // 64) of one selection."""
    words = np.zeros((NB + 63) // 64, dtype=np.uint64)
    for kb in sel.selected:
        words[kb // 64] |= np.uint64(1) << np.uint64(kb % 64)
    return words


# ---------------------------------------------------------------------------
# Step 5 -- attention restricted to the selected blocks (block-sparse attention).
# ---------------------------------------------------------------------------
def block_sparse_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, B: int,
                           causal: bool, qb: int, kblocks: Iterable[int]) -> np.ndarray:
    """Output rows of query block qb: softmax(q k^T / sqrt(d)) over the keys of
    the blocks `kblocks` (and j <= i when causal), applied to V.  float64 [B][d]."""
    d = Q.shape[1]
    q = Q[qb * B:(qb + 1) * B]
    kbs = sorted(set(int(k) for k in kblocks))
    if not kbs:
        return np.zeros((B, V.shape[1]))
    keys = np.concatenate([np.arange(kb * B, (kb + 1) * B) for kb in kbs])
    logits = (q @ K[keys].T) / math.sqrt(d)
    if causal:
        i = np.arange(qb * B, (qb + 1) * B)[:, None]
        logits = np.where(keys[None, :] > i, -np.inf, logits)
    m = logits.max(axis=1, keepdims=True)
    live = np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(logits - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ V[keys]) / np.where(den > 0, den, 1.0)
    out[~live] = 0.0
    return out


def full_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, B: int, causal: bool,
                   qb: int) -> np.ndarray:
    """Dense attention for the rows of query block qb (all keys, j <= i if causal)."""
    NB = Q.shape[0] // B
    return block_sparse_attention(Q, K, V, B, causal, qb, range(qb + 1 if causal else NB))


# ---------------------------------------------------------------------------
# Video DiT warm-up policy (chapterpal.com Knowl 4, "Full-Attention Denoising
# Warmup"; papercache.org summary, video generation experiment): dense
# attention for the first `warmup` denoising steps (5 of 50 on the pages),
# XAttention afterwards.
# ---------------------------------------------------------------------------
def dit_step_is_dense(step: int, warmup: int = 5) -> bool:
    """Denoising steps count from 0; steps 0 .. warmup-1 are dense."""
    return step < warmup


def dit_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, S: int, B: int, tau: float,
                  step: int, warmup: int, qb: int, causal: bool = False) -> np.ndarray:
    """Output rows of query block qb at denoising step `step`: full attention
    during the warm-up, else threshold-selected block-sparse attention."""
    if dit_step_is_dense(step, warmup):
        return full_attention(Q, K, V, B, causal, qb)
    NB = Q.shape[0] // B
    row = block_scores(Q, K, S, B, causal, qblocks=[qb])[0]
    sel = find_blocks(row, qb + 1 if causal else NB, tau)
    return block_sparse_attention(Q, K, V, B, causal, qb, sel.selected)


def dit_run_density(sparse_density: float, steps: int = 50, warmup: int = 5) -> float:
    """Share of attention blocks computed over a whole generation run: dense
    steps count as density 1."""
    n_dense = sum(1 for t in range(steps) if dit_step_is_dense(t, warmup))
    return (n_dense + (steps - n_dense) * sparse_density) / steps


# ---------------------------------------------------------------------------
# Minimum threshold prediction (papercache.org summary, section 2.3 "minimum
# threshold prediction"; chapterpal.com Knowl 3): per-head thresholds chosen by
# dynamic programming over threshold-reduction steps, each step multiplying a
# head's threshold by 0.9.  The pages' performance P(h, m) is downstream model
# accuracy; here it is a proxy, minus the sum over heads of the relative
# squared error of the head's sparse output against its dense output.
# ---------------------------------------------------------------------------
def head_rel_sq_error(O_sparse: np.ndarray, O_dense: np.ndarray) -> float:
    """sum (O_sparse - O_dense)^2 / sum O_dense^2 over one head's [L][d] output."""
    a = np.asarray(O_sparse, dtype=np.float64)
    b = np.asarray(O_dense, dtype=np.float64)
    den = float((b * b).sum())
    return float(((a - b) ** 2).sum()) / den if den > 0 else 0.0


def tau_levels(tau0: float, levels: int) -> List[float]:
    """Threshold after k reduction steps, k = 0 .. levels: tau0 * 0.9^k."""
    t, out = float(tau0), []
    for _ in range(levels + 1):
        out.append(t)
        t *= 0.9
    return out


def tau_dp(err: np.ndarray, steps: int) -> Tuple[List[int], float]:
    """Distribute exactly `steps` reduction steps over the heads.

    err[h][k]: proxy error of head h after k steps (k = 0 .. R).  D[h][m] is
    the best performance (minus the summed error) of heads 0 .. h-1 having
    taken m steps in total; head h either keeps its level-0 threshold or takes
    k steps on top of the best state with m - k steps over the heads before it
    -- with R = 1 exactly the printed recurrence D[h][m] = max(D[h-1][m],
    P(h, m)).  Ties keep the smaller k for the later head.  Returns the levels
    per head (traced back from D[H][steps]) and that best value."""
    err = np.asarray(err, dtype=np.float64)
    H, R1 = err.shape
    R = R1 - 1
    assert 0 <= steps <= H * R, "steps must lie in [0, H*R]"
    D = np.full((H + 1, steps + 1), -np.inf)
    take = np.zeros((H + 1, steps + 1), dtype=np.int64)
    D[0, 0] = 0.0
    for h in range(1, H + 1):
        for m in range(steps + 1):
            for k in range(0, min(R, m) + 1):
                if D[h - 1, m - k] == -np.inf:
                    continue
                cand = D[h - 1, m - k] - err[h - 1, k]
                if cand > D[h, m]:
                    D[h, m] = cand
                    take[h, m] = k
    levels, m = [0] * H, steps
    for h in range(H, 0, -1):
        levels[h - 1] = int(take[h, m])
        m -= levels[h - 1]
    return levels, float(D[H, steps])
