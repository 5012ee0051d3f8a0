"""The mask comparison rule of the GPU parity tests, checked on the CPU with
hand-built rows: outside the tau band only identical selections pass, a
near-tie at the cut included; inside it the cut may move by one block and
near-tied blocks may swap, but the set must stay a top set of the oracle's
ranking (find_blocks of the papercache.org summary, section 2.2: the
shortest prefix of the ranking whose mass is >= tau)."""
import numpy as np

import oracle as O
from parity import TAU_BAND, classify_rows, in_tau_band, in_tie_band


def _row(scores, tau):
    scores = np.asarray(scores, dtype=np.float64)
    sel = O.find_blocks(scores, len(scores), tau)
    return sel, scores[sel.order]


def _classify(scores, tau, gset):
    sel, srt = _row(scores, tau)
    return classify_rows([sel], [srt], [list(gset)], [tau], ["row"])


# ranking 3 (0.4), 1 (0.3), 0 (0.2), 2 (0.1); prefixes 0.4, 0.7, 0.9, 1.0
SCORES = [0.2, 0.3, 0.1, 0.4]


def test_identical_selection_passes():
    rep = _classify(SCORES, 0.65, [1, 3])
    assert rep.equal == 1 and not rep.failures


def test_mismatch_outside_tau_band_fails():
    # tau = 0.65: k* = 2, prefixes 0.4 / 0.7 are far from tau
    for gset in ([3], [1, 3, 0], [0, 3], [1, 2]):
        rep = _classify(SCORES, 0.65, gset)
        assert len(rep.failures) == 1, gset
        assert rep.tau_band == 0


def test_tau_band_allows_only_neighbouring_prefixes():
    tau = 0.7 + TAU_BAND / 2          # P_2 = 0.7 lies within the band -> k* = 3
    sel, srt = _row(SCORES, tau)
    assert sel.kstar == 3 and in_tau_band(sel, tau)
    assert not _classify(SCORES, tau, [1, 3]).failures            # prefix of length 2
    assert not _classify(SCORES, tau, [0, 1, 2, 3]).failures      # prefix of length 4
    rep = _classify(SCORES, tau, [0, 1, 2])                      # size 3, wrong set
    assert len(rep.failures) == 1 and rep.tau_band == 1
    rep = _classify(SCORES, tau, [3])                            # cut moved by two
    assert len(rep.failures) == 1


def test_near_tie_at_the_cut_is_not_exempt():
    # blocks 0 and 1 differ by 1e-6 relative; tau = 0.2 keeps only block 0
    scores = [0.3, 0.3 * (1 - 1e-6), 0.25, 0.15 + 0.3e-6]
    sel, srt = _row(scores, 0.2)
    assert sel.kstar == 1 and list(sel.selected) == [0]
    assert in_tie_band(srt, sel) and not in_tau_band(sel, 0.2)
    rep = _classify(scores, 0.2, [1])
    assert len(rep.failures) == 1 and rep.tie_band == 1
    assert "tie band True" in rep.failures[0]


def test_tau_band_accepts_a_near_tie_swap_but_not_a_real_one():
    # blocks 1 and 2 differ by 1e-6 relative; tau sits 5e-5 above P_1
    scores = np.array([0.5, 0.2, 0.2 * (1 - 1e-6), 0.1 + 0.2e-6])
    tau = 0.5 + 5e-5
    sel, srt = _row(scores, tau)
    assert sel.kstar == 2 and list(sel.selected) == [0, 1]
    assert in_tau_band(sel, tau) and in_tie_band(srt, sel)
    rep = _classify(scores, tau, [0, 2])          # near-tied swap at the cut
    assert not rep.failures and rep.tau_band_moved == 1
    rep = _classify(scores, tau, [0, 3])          # block 3 is no near-tie of 1
    assert len(rep.failures) == 1
    rep = _classify(scores, tau, [1, 2])          # drops the top block
    assert len(rep.failures) == 1
