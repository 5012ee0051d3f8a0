"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the literal
reshape of Algorithm 1, brute force over tiny inputs, printed or hand-derived
worked values (tests/golden), closed forms and invariants.  No GPU needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- Algorithm 1 written literally (papercache.org summary, section 2.2) ------
def literal_algorithm1_product(Q, K, B, S, b):
    """Q_reshaped K_reshaped^T of query block b, built as Algorithm 1 describes:
    query slices taken with phase S-1 down to 0 and key slices with phase 0 up
    to S-1, each appended along the feature axis."""
    q_slice = Q[b * B:(b + 1) * B]
    q_res = np.concatenate([q_slice[i::S] for i in range(S - 1, -1, -1)], axis=1)
    k_res = np.concatenate([K[i::S] for i in range(S)], axis=1)
    return q_res @ k_res.T


@pytest.mark.parametrize("S,B", [(1, 1), (1, 4), (2, 2), (2, 4), (2, 8), (4, 4), (4, 8),
                                 (4, 16), (8, 8), (8, 16), (8, 32)])
def test_antidiagonal_sums_equal_literal_reshape(S, B):
    rng = np.random.default_rng(100 + 10 * S + B)
    L, d = 32, 3
    Q = rng.integers(-9, 10, size=(L, d)).astype(np.float64)
    K = rng.integers(-9, 10, size=(L, d)).astype(np.float64)
    A = O.antidiagonal_sums(Q, K, S)
    for b in range(L // B):
        lit = literal_algorithm1_product(Q, K, B, S, b)
        np.testing.assert_array_equal(A[b * B // S:(b + 1) * B // S], lit)


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_antidiagonal_sums_brute_force_tile_antidiagonals(S):
    """Q = M, K = I makes Q K^T = M: A[R, c] must be the sum of M over the SxS
    tile's sampled set {(i, j): (i + j + 1) mod S == 0}, by explicit loops."""
    rng = np.random.default_rng(7 + S)
    L = 4 * S * 2
    M = rng.integers(-50, 51, size=(L, L)).astype(np.float64)
    A = O.antidiagonal_sums(M, np.eye(L), S)
    Lr = L // S
    for R in range(Lr):
        for c in range(Lr):
            tot = 0.0
            for i in range(R * S, (R + 1) * S):
                for j in range(c * S, (c + 1) * S):
                    if (i + j + 1) % S == 0:
                        tot += M[i, j]
            assert A[R, c] == tot


def _perm(S, kind, seed=0):
    if kind == "antidiagonal":
        return [S - 1 - a for a in range(S)]
    if kind == "diagonal":
        return list(range(S))
    return [int(x) for x in np.random.default_rng(seed).permutation(S)]


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("kind", ["antidiagonal", "diagonal", "random"])
def test_pattern_sums_brute_force_tile_samples(S, kind):
    """Q = M, K = I: A[R, c] is the sum of M over the tile entries (RS + a,
    cS + phase[a]), by explicit loops; the antidiagonal phase reproduces
    antidiagonal_sums exactly."""
    rng = np.random.default_rng(31 + S)
    L = 4 * S * 2
    M = rng.integers(-50, 51, size=(L, L)).astype(np.float64)
    ph = _perm(S, kind, seed=S)
    A = O.pattern_sums(M, np.eye(L), S, ph)
    for R in range(L // S):
        for c in range(L // S):
            tot = 0.0
            for a in range(S):
                tot += M[R * S + a, c * S + ph[a]]
            assert A[R, c] == tot
    if kind == "antidiagonal":
        np.testing.assert_array_equal(A, O.antidiagonal_sums(M, np.eye(L), S))


@pytest.mark.parametrize("S", [2, 4, 8])
def test_diagonal_pattern_samples_every_sth_diagonal(S):
    """The diagonal pattern sums exactly the entries with (i - j) mod S == 0,
    which include the main diagonal (i == j) that the antidiagonal pattern
    never samples for even S."""
    rng = np.random.default_rng(5 + S)
    L = 6 * S
    M = rng.integers(-20, 21, size=(L, L)).astype(np.float64)
    A = O.pattern_sums(M, np.eye(L), S, list(range(S)))
    for R in range(L // S):
        for c in range(L // S):
            tot = sum(M[i, j] for i in range(R * S, (R + 1) * S)
                      for j in range(c * S, (c + 1) * S) if (i - j) % S == 0)
            assert A[R, c] == tot


@pytest.mark.parametrize("kind", ["antidiagonal", "diagonal", "random"])
def test_pattern_block_scores_rows_sum_to_one(kind):
    rng = np.random.default_rng(9)
    L, d, S, B = 512, 16, 8, 64
    Q, K = rng.standard_normal((L, d)) * 2, rng.standard_normal((L, d)) * 2
    ph = _perm(S, kind, seed=3)
    for causal in (True, False):
        sc = O.block_scores(Q, K, S, B, causal, phase=ph)
        np.testing.assert_allclose(sc.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            assert np.all(np.triu(sc, 1) == 0)
        if kind == "antidiagonal":
            np.testing.assert_array_equal(sc, O.block_scores(Q, K, S, B, causal))


def test_pattern_rejects_non_permutation():
    with pytest.raises(AssertionError):
        O.pattern_sums(np.zeros((8, 2)), np.zeros((8, 2)), 4, [0, 1, 1, 2])


@pytest.mark.parametrize("S,B", [(2, 8), (4, 8), (4, 16), (8, 16), (8, 64)])
def test_sampled_set_invariants(S, B):
    """Which entries of Q K^T the scores sum: every key is hit exactly once per
    reshaped row (every vertical line is met), every token B/S times per
    block, and for even S only odd offsets i - j are sampled."""
    L = 2 * B
    hit = np.zeros((L, L), dtype=np.int64)
    for i in range(L):
        for j in range(L):
            M = np.zeros((L, L))
            M[i, j] = 1.0
            A = O.antidiagonal_sums(M, np.eye(L), S)
            hit[i, j] = int(A[i // S, j // S])
            assert A.sum() == hit[i, j]
    for R in range(L // S):
        np.testing.assert_array_equal(hit[R * S:(R + 1) * S].sum(axis=0), 1)
    for qb in range(L // B):
        for kb in range(L // B):
            tile = hit[qb * B:(qb + 1) * B, kb * B:(kb + 1) * B]
            np.testing.assert_array_equal(tile.sum(axis=0), B // S)
            np.testing.assert_array_equal(tile.sum(axis=1), B // S)
    if S % 2 == 0:
        ii, jj = np.nonzero(hit)
        assert np.all((ii - jj) % 2 == 1)


def test_page5_qk_worked_example():
    g = _golden("page5_qk.json")
    Q, K = np.array(g["Q"]), np.array(g["K"])
    # S = 1: the reshape is the identity and the scores are Q K^T itself, which
    # fixes the orientation of the product (rows: queries, columns: keys).
    np.testing.assert_array_equal(O.antidiagonal_sums(Q, K, 1), np.array(g["QKt"]))


def test_softmax_scale_closed_form():
    g = _golden("scale_two_columns.json")
    Q, K = np.array(g["Q"]), np.array(g["K"])
    A = O.antidiagonal_sums(Q, K, g["S"])
    np.testing.assert_array_equal(A[0], [0.0, Q[0, 0]])
    P = O.approx_attention(A, g["d"], g["S"], causal=False, row0=0)
    np.testing.assert_allclose(P[0], g["row0_probs"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_and_causal_mask(causal):
    rng = np.random.default_rng(3)
    L, d, S = 256, 16, 4
    Q, K = rng.standard_normal((L, d)) * 3, rng.standard_normal((L, d)) * 3
    A = O.antidiagonal_sums(Q, K, S, range(8, 40))
    P = O.approx_attention(A, d, S, causal, row0=8)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(P >= 0)
    if causal:
        for r in range(P.shape[0]):
            R = 8 + r
            assert np.all(P[r, R + 1:] == 0.0)
            assert P[r, R] > 0.0          # the diagonal entry keeps its antidiagonal


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,B", [(2, 8), (4, 16), (8, 16), (8, 64)])
def test_block_scores_rows_sum_to_one(causal, S, B):
    rng = np.random.default_rng(11)
    L, d = 256, 8
    Q, K = rng.standard_normal((L, d)) * 2, rng.standard_normal((L, d)) * 2
    sc = O.block_scores(Q, K, S, B, causal)
    np.testing.assert_allclose(sc.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    if causal:
        NB = L // B
        for qb in range(NB):
            assert np.all(sc[qb, qb + 1:] == 0.0)


def _naive_attention_weights(Q, K, causal):
    """Textbook softmax(q k^T / sqrt(d)) weights by explicit loops."""
    L, d = Q.shape
    W = np.zeros((L, L))
    for i in range(L):
        logits = []
        for j in range(L):
            if causal and j > i:
                logits.append(None)
            else:
                logits.append(sum(Q[i, t] * K[j, t] for t in range(d)) / math.sqrt(d))
        m = max(x for x in logits if x is not None)
        den = sum(math.exp(x - m) for x in logits if x is not None)
        for j in range(L):
            if logits[j] is not None:
                W[i, j] = math.exp(logits[j] - m) / den
    return W


@pytest.mark.parametrize("causal", [False, True])
def test_stride_one_is_exact_attention_mass(causal):
    """S = 1: A_approx is exact attention, so a block score is (1/B) times the
    exact attention mass of the block."""
    rng = np.random.default_rng(5)
    L, d, B = 24, 4, 4
    Q, K = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    W = _naive_attention_weights(Q, K, causal)
    sc = O.block_scores(Q, K, 1, B, causal)
    NB = L // B
    for qb in range(NB):
        for kb in range(NB):
            want = W[qb * B:(qb + 1) * B, kb * B:(kb + 1) * B].sum() / B
            assert abs(sc[qb, kb] - want) < 1e-13


def test_block_equals_stride_scores_are_probabilities():
    """B == S: each query block is one reshaped row, so the block scores are
    the reshaped softmax row itself."""
    rng = np.random.default_rng(6)
    L, d, S = 64, 4, 4
    Q, K = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    for causal in (False, True):
        P = O.approx_attention(O.antidiagonal_sums(Q, K, S), d, S, causal, 0)
        np.testing.assert_allclose(O.block_scores(Q, K, S, S, causal), P, rtol=0, atol=1e-15)


def test_block_scores_chunking_invariant():
    rng = np.random.default_rng(9)
    L, d, S, B = 512, 8, 4, 32
    Q, K = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    full = O.block_scores(Q, K, S, B, True, chunk=64)
    one = O.block_scores(Q, K, S, B, True, chunk=1)
    some = O.block_scores(Q, K, S, B, True, qblocks=[3, 4, 5, 9, 15])
    np.testing.assert_allclose(full, one, rtol=0, atol=1e-15)
    np.testing.assert_allclose(full[[3, 4, 5, 9, 15]], some, rtol=0, atol=1e-15)


# --- find_blocks ------------------------------------------------------------
@pytest.mark.parametrize("trial", range(60))
def test_find_blocks_minimal_by_subset_enumeration(trial):
    rng = np.random.default_rng(1000 + trial)
    n = int(rng.integers(1, 11))
    mass = rng.dirichlet(np.full(n, float(rng.choice([0.3, 1.0, 5.0]))))
    if trial % 5 == 0:                      # force exact ties
        mass = np.round(mass * 8) / 8
        mass = mass / mass.sum()
    tau = float(rng.choice([0.5, 0.8, 0.9, 0.95, rng.uniform(0.05, 1.0)]))
    sel = O.find_blocks(mass, n, tau)
    best = None
    for k in range(1, n + 1):
        if any(sum(mass[list(c)]) >= tau for c in itertools.combinations(range(n), k)):
            best = k
            break
    assert sel.kstar == (best if best is not None else n)
    # the chosen set is the top-k* by (mass desc, index asc)
    ranked = sorted(range(n), key=lambda j: (-mass[j], j))
    assert sorted(ranked[:sel.kstar]) == list(sel.selected)


def test_find_blocks_uses_greater_or_equal():
    mass = np.array([0.5, 0.25, 0.25])   # exact in binary
    assert O.find_blocks(mass, 3, 0.75).kstar == 2
    assert O.find_blocks(mass, 3, 0.5).kstar == 1
    assert list(O.find_blocks(mass, 3, 0.75).selected) == [0, 1]


def test_tie_break_uniform_scores():
    """Q = 0, non-causal: every score is 1/NB (exact for NB = 16), and tau = 0.5
    keeps the 8 lowest key blocks."""
    L, d, S, B = 256, 8, 4, 16
    Q = np.zeros((L, d))
    K = np.random.default_rng(2).standard_normal((L, d))
    sc = O.block_scores(Q, K, S, B, causal=False)
    assert np.all(sc == 1.0 / 16)
    for sel in O.select_all(sc, False, 0.5):
        assert list(sel.selected) == list(range(8))


def test_tau_one_selects_every_causal_block():
    rng = np.random.default_rng(4)
    L, d, S, B = 256, 8, 4, 16
    Q, K = rng.standard_normal((L, d)) * 4, rng.standard_normal((L, d)) * 4
    sc = O.block_scores(Q, K, S, B, causal=True)
    for qb, sel in enumerate(O.select_all(sc, True, 1.0)):
        assert list(sel.selected) == list(range(qb + 1))
        words = O.to_mask(sel, L // B)
        assert int(words[0]) == (1 << (qb + 1)) - 1


# --- Top-K / Top-Ratio cut rules (ablation "selection strategy") ------------
@pytest.mark.parametrize("trial", range(40))
def test_topk_is_a_best_k_subset_by_enumeration(trial):
    """For every k, the Top-K set has the largest total mass of all k-subsets
    (brute force), and it is the one the ranking picks: every selected block
    outranks every unselected one by (mass desc, index asc)."""
    rng = np.random.default_rng(3000 + trial)
    n = int(rng.integers(1, 10))
    mass = rng.dirichlet(np.full(n, float(rng.choice([0.3, 1.0, 5.0]))))
    if trial % 4 == 0:                      # exact ties
        mass = np.round(mass * 6) / 6
    for k in range(1, n + 1):
        sel = O.find_blocks_topk(mass, n, k)
        assert sel.kstar == k and len(sel.selected) == k
        best = max(sum(mass[list(c)]) for c in itertools.combinations(range(n), k))
        assert math.isclose(float(mass[sel.selected].sum()), best, rel_tol=0, abs_tol=1e-12)
        chosen = set(int(j) for j in sel.selected)
        for a in chosen:
            for b in set(range(n)) - chosen:
                assert (mass[a] > mass[b]) or (mass[a] == mass[b] and a < b)


def test_topk_clamps_to_valid_blocks():
    mass = np.array([0.1, 0.4, 0.2, 0.3])
    assert list(O.find_blocks_topk(mass, 4, 10).selected) == [0, 1, 2, 3]
    assert list(O.find_blocks_topk(mass, 2, 5).selected) == [0, 1]     # causal row: 2 valid
    assert list(O.find_blocks_topk(mass, 4, 1).selected) == [1]
    assert list(O.find_blocks_topk(mass, 4, 2).selected) == [1, 3]


def test_topk_agrees_with_threshold_cut():
    """Cutting the ranking at the threshold rule's k* gives the threshold
    rule's set (the two rules differ only in where the ranked prefix ends)."""
    rng = np.random.default_rng(11)
    L, d, S, B = 512, 16, 4, 32
    Q, K = rng.standard_normal((L, d)) * 3, rng.standard_normal((L, d)) * 3
    sc = O.block_scores(Q, K, S, B, causal=True)
    for qb in range(sc.shape[0]):
        for tau in (0.3, 0.8, 0.95):
            thr = O.find_blocks(sc[qb], qb + 1, tau)
            top = O.find_blocks_topk(sc[qb], qb + 1, thr.kstar)
            assert list(top.selected) == list(thr.selected)


@pytest.mark.parametrize("n,ratio,want", [
    (100, 0.27, 27),      # float32(0.27) * 100 = 27.000001..., not 28
    (1024, 0.27, 276),    # 276.48
    (2, 0.27, 1), (1, 0.27, 1), (1, 1e-6, 1),     # at least one block
    (10, 1.0, 10), (3, 0.5, 2), (7, 0.5, 4),      # halves round up
    (8192, 0.27, 2212),   # 2211.84
])
def test_topratio_count_closed_form(n, ratio, want):
    assert O.topratio_count(n, ratio) == want
    assert O.find_blocks_topratio(np.linspace(1, 2, n), n, ratio).kstar == want


def test_topk_tie_break_uniform_scores():
    """Q = 0: every block scores 1/NB; Top-K keeps the k lowest key blocks."""
    L, d, S, B = 256, 8, 4, 16
    Q = np.zeros((L, d))
    K = np.random.default_rng(2).standard_normal((L, d))
    sc = O.block_scores(Q, K, S, B, causal=False)
    for qb in range(sc.shape[0]):
        assert list(O.find_blocks_topk(sc[qb], 16, 5).selected) == [0, 1, 2, 3, 4]
        assert list(O.find_blocks_topratio(sc[qb], 16, 0.25).selected) == [0, 1, 2, 3]


# --- block-sparse attention -------------------------------------------------
def _naive_attention(Q, K, V, causal, allowed=None):
    L, d = Q.shape
    out = np.zeros((L, V.shape[1]))
    for i in range(L):
        logits = {}
        for j in range(K.shape[0]):
            if causal and j > i:
                continue
            if allowed is not None and j not in allowed:
                continue
            logits[j] = sum(Q[i, t] * K[j, t] for t in range(d)) / math.sqrt(d)
        if not logits:
            continue
        m = max(logits.values())
        den = sum(math.exp(x - m) for x in logits.values())
        for j, x in logits.items():
            out[i] += math.exp(x - m) / den * V[j]
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_tau_one_sparse_equals_naive_full_attention(causal):
    rng = np.random.default_rng(21)
    L, d, S, B = 32, 4, 2, 8
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    sc = O.block_scores(Q, K, S, B, causal)
    want = _naive_attention(Q, K, V, causal)
    for qb, sel in enumerate(O.select_all(sc, causal, 1.0)):
        got = O.block_sparse_attention(Q, K, V, B, causal, qb, sel.selected)
        np.testing.assert_allclose(got, want[qb * B:(qb + 1) * B], rtol=0, atol=1e-12)
        np.testing.assert_allclose(O.full_attention(Q, K, V, B, causal, qb),
                                   want[qb * B:(qb + 1) * B], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_attention_restricted_to_selected_blocks(causal):
    rng = np.random.default_rng(22)
    L, d, B = 32, 3, 8
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    qb = 3
    for kbs in ([1], [0, 2], [3], [1, 3]):
        allowed = set(j for kb in kbs for j in range(kb * B, (kb + 1) * B))
        want = _naive_attention(Q, K, V, causal, allowed)[qb * B:(qb + 1) * B]
        got = O.block_sparse_attention(Q, K, V, B, causal, qb, kbs)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_single_key_row_copies_value():
    """A causal row whose only visible key is itself outputs that key's V."""
    rng = np.random.default_rng(23)
    L, d, B = 16, 4, 8
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    out = O.block_sparse_attention(Q, K, V, B, True, 1, [1])
    np.testing.assert_allclose(out[0], V[8], rtol=0, atol=1e-15)
    # no selected block: rows output 0
    assert np.all(O.block_sparse_attention(Q, K, V, B, True, 1, []) == 0.0)


# --- video DiT warm-up policy --------------------------------------------------
def test_dit_schedule_first_five_of_fifty_dense():
    dense = [t for t in range(50) if O.dit_step_is_dense(t, 5)]
    assert dense == [0, 1, 2, 3, 4]
    # density over the run: dense steps count as 1
    assert math.isclose(O.dit_run_density(0.4, 50, 5), (5 + 45 * 0.4) / 50)
    assert O.dit_run_density(1.0) == 1.0
    assert O.dit_run_density(0.0, 50, 5) == 0.1
    # sparsity over the run stays above 50% exactly when the sparse steps keep < 4/9 of blocks
    assert O.dit_run_density(4 / 9 - 1e-9) < 0.5 < O.dit_run_density(4 / 9 + 1e-9)


def test_dit_attention_dense_steps_and_tau_one_are_naive_attention():
    rng = np.random.default_rng(21)
    L, d, S, B = 32, 4, 2, 8
    Q, K, V = (rng.standard_normal((L, d)) for _ in range(3))
    naive = _naive_attention(Q, K, V, causal=False)
    for qb in range(L // B):
        rows = slice(qb * B, (qb + 1) * B)
        for step in range(5):             # warm-up steps: dense whatever tau says
            np.testing.assert_allclose(O.dit_attention(Q, K, V, S, B, 0.3, step, 5, qb),
                                       naive[rows], rtol=0, atol=1e-12)
        np.testing.assert_allclose(O.dit_attention(Q, K, V, S, B, 1.0, 7, 5, qb), naive[rows],
                                   rtol=0, atol=1e-12)


def test_dit_attention_sparse_step_is_restricted_attention():
    """After the warm-up, a query block attends to exactly the keys of its
    selected blocks: equal to naive attention over those keys."""
    rng = np.random.default_rng(22)
    L, d, S, B = 32, 4, 2, 8
    Q, K, V = (rng.standard_normal((L, d)) * 2 for _ in range(3))
    sc = O.block_scores(Q, K, S, B, causal=False)
    for qb in range(L // B):
        sel = O.find_blocks(sc[qb], L // B, 0.6)
        allowed = {j for kb in sel.selected for j in range(kb * B, (kb + 1) * B)}
        want = _naive_attention(Q, K, V, causal=False, allowed=allowed)[qb * B:(qb + 1) * B]
        np.testing.assert_allclose(O.dit_attention(Q, K, V, S, B, 0.6, 5, 5, qb), want,
                                   rtol=0, atol=1e-12)


# --- minimum threshold prediction (per-head tau DP) ---------------------------
def _monotone_errors(rng, H, R):
    inc = rng.exponential(1.0, size=(H, R + 1))
    inc[:, 0] = rng.uniform(0, 0.1, size=H)
    return np.cumsum(inc, axis=1)


@pytest.mark.parametrize("trial", range(25))
def test_tau_dp_is_optimal_by_enumeration(trial):
    rng = np.random.default_rng(4000 + trial)
    H, R = int(rng.integers(1, 6)), int(rng.integers(1, 4))
    err = _monotone_errors(rng, H, R)
    if trial % 5 == 0:
        err = np.round(err * 2) / 2          # exact ties
    for steps in range(H * R + 1):
        levels, best = O.tau_dp(err, steps)
        assert sum(levels) == steps and all(0 <= k <= R for k in levels)
        assert math.isclose(-sum(err[h, k] for h, k in enumerate(levels)), best,
                            rel_tol=0, abs_tol=1e-12)
        brute = max(-sum(err[h, k] for h, k in enumerate(ks))
                    for ks in itertools.product(range(R + 1), repeat=H) if sum(ks) == steps)
        assert math.isclose(best, brute, rel_tol=0, abs_tol=1e-12)


def test_tau_dp_one_step_per_head_takes_the_cheapest_heads():
    """R = 1 (the printed recurrence): the m reduced heads are those whose
    error grows least from one step."""
    rng = np.random.default_rng(44)
    H = 12
    err = _monotone_errors(rng, H, 1)
    inc = err[:, 1] - err[:, 0]
    for m in range(H + 1):
        levels, _ = O.tau_dp(err, m)
        assert sorted(h for h in range(H) if levels[h]) == sorted(np.argsort(inc)[:m].tolist())


def test_tau_dp_extremes_and_levels():
    err = _monotone_errors(np.random.default_rng(3), 6, 3)
    assert O.tau_dp(err, 0)[0] == [0] * 6
    assert O.tau_dp(err, 18)[0] == [3] * 6
    t = O.tau_levels(0.9, 3)
    np.testing.assert_allclose(t, [0.9, 0.81, 0.729, 0.6561], rtol=0, atol=1e-15)
    # with one step per head (R = 1, steps = H) every head takes it: the mean
    # threshold goes from 0.9 to 0.81 (the pages: from 0.9 to about 0.8)
    lv, _ = O.tau_dp(err[:, :2], 6)
    assert lv == [1] * 6
    assert math.isclose(float(np.mean([O.tau_levels(0.9, 1)[k] for k in lv])), 0.81)


def test_head_rel_sq_error_properties():
    rng = np.random.default_rng(8)
    b = rng.standard_normal((64, 16))
    a = b + 0.01 * rng.standard_normal((64, 16))
    assert O.head_rel_sq_error(b, b) == 0.0
    assert O.head_rel_sq_error(np.zeros_like(b), b) == 1.0
    assert math.isclose(O.head_rel_sq_error(3 * a, 3 * b), O.head_rel_sq_error(a, b), rel_tol=1e-12)
    manual = sum(((a - b) ** 2).flat) / sum((b ** 2).flat)
    assert math.isclose(O.head_rel_sq_error(a, b), manual, rel_tol=1e-12)


def test_to_mask_multi_word_layout():
    """Mask words for NB > 64 (bit kb % 64 of word kb // 64), with the words
    written out by hand: blocks {0, 63} -> word 0, {64, 65, 127} -> word 1,
    {128} -> word 2, {199} -> word 3 (bit 7)."""
    sel = O.Selection(selected=np.array([0, 63, 64, 65, 127, 128, 199]), kstar=7,
                      order=np.array([0, 63, 64, 65, 127, 128, 199]), csum=np.ones(7), n_valid=200)
    words = O.to_mask(sel, 200)
    assert words.dtype == np.uint64 and words.shape == (4,)
    assert [int(x) for x in words] == [0x8000000000000001, 0x8000000000000003, 0x1, 0x80]
    # and against one big integer holding bit kb for every selected block
    big = sum(1 << int(kb) for kb in sel.selected)
    assert [int(x) for x in words] == [(big >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
    # NB = 65: two words, the second holding only block 64
    sel65 = O.find_blocks(np.r_[np.zeros(64), 1.0], 65, 0.5)
    assert list(sel65.selected) == [64]
    assert [int(x) for x in O.to_mask(sel65, 65)] == [0, 1]
