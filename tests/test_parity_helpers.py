"""CPU tests of the selection comparison used by the GPU parity tests: the
near-tie exemption applies only where the gate had a choice, with the -1
padding in the oracle's slots, and only on a near-tie of the fp32 scores."""

import numpy as np

from oracle import select_blocks
from tests.parity import compare_selection, near_tie


def _setup(zero_q):
    N, H, D, B, topk = 64, 1, 8, 8, 3
    rng = np.random.default_rng(901)
    q = rng.standard_normal((N, H, D)).astype(np.float32)
    k = rng.standard_normal((N, H, D)).astype(np.float32)
    if zero_q:
        q[:] = 0.0
    ref, _ = select_blocks(q, k, B, topk)
    return q, k, B, topk, ref


def test_identical_selection_passes():
    q, k, B, topk, ref = _setup(False)
    r = compare_selection(ref.copy(), ref, q, k, B, topk)
    assert r["mismatch"] == 0 and not r["bad"]


def test_exact_tie_is_exempt():
    """q = 0: every score is 0, any valid choice of past blocks is a tie."""
    q, k, B, topk, ref = _setup(True)
    gpu = ref.copy()
    t = 40                                    # block 5: blocks 0..4 compete for two slots
    assert list(ref[0, t]) == [0, 1, 5]
    gpu[0, t] = [2, 3, 5]
    r = compare_selection(gpu, ref, q, k, B, topk)
    assert r["mismatch"] == 1 and r["exempt"] == 1 and r["exempt_rowmax"] == 1 and not r["bad"]


def test_misplaced_padding_is_rejected():
    q, k, B, topk, ref = _setup(True)
    gpu = ref.copy()
    t = 10                                    # block 1: fewer eligible blocks than top_k, padded
    assert list(ref[0, t]) == [0, 1, -1]
    gpu[0, t] = [0, -1, 1]
    r = compare_selection(gpu, ref, q, k, B, topk)
    assert r["mismatch"] == 1 and r["exempt"] == 0 and len(r["bad"]) == 1 and len(r["bad_rowmax"]) == 1


def test_padding_in_a_ranked_row_is_rejected():
    q, k, B, topk, ref = _setup(True)
    gpu = ref.copy()
    gpu[0, 40] = [0, -1, 5]
    r = compare_selection(gpu, ref, q, k, B, topk)
    assert len(r["bad"]) == 1


def test_unranked_row_must_match():
    """Block 2 with top-3: every block 0..2 is kept, there is no gate decision
    (and so no tie) to exempt, even where all scores are equal."""
    q, k, B, topk, ref = _setup(True)
    for row in ([0, 2, 2], [1, 2, 0], [0, 1, 1]):
        gpu = ref.copy()
        gpu[0, 17] = row
        r = compare_selection(gpu, ref, q, k, B, topk)
        assert r["mismatch"] == 1 and len(r["bad"]) == 1 and r["exempt"] == 0, row


def test_clear_score_gap_is_rejected():
    q, k, B, topk, ref = _setup(False)
    gpu = ref.copy()
    t = 63                                    # block 7: blocks 0..6 compete
    past = [int(x) for x in ref[0, t] if x != 7]
    other = [b for b in range(7) if b not in past][0]
    gpu[0, t] = sorted([past[0], other]) + [7]
    r = compare_selection(gpu, ref, q, k, B, topk)
    assert r["mismatch"] == 1 and len(r["bad"]) == 1 and len(r["bad_rowmax"]) == 1


def test_pairwise_rule_is_stricter_than_row_max():
    """Two small scores 5e-5 apart in a row whose largest |score| is 1: a tie
    under the row-max denominator, not under the pair's own magnitude."""
    g = np.array([1.0, 1e-3, 1.05e-3, -0.5])
    assert near_tie(g, [2], [1], j=4) == (False, True)
    # Within 1e-4 of their own magnitude: a tie under both rules.
    g2 = np.array([1.0, 0.25, 0.25 * (1 + 5e-5), -0.5])
    assert near_tie(g2, [2], [1], j=4) == (True, True)
    # Different set sizes are never a tie.
    assert near_tie(g2, [1, 2], [1], j=4) == (False, False)
