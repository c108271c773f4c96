"""The acceptance rule (tests/parity.py) is not vacuous (no GPU).

Each case feeds ``check`` the oracle's own answer with one planted error and
requires a failure; the untouched answer, and a pick that lies inside the
oracle's top-two gap, must pass.  The planted errors are the ones a broken
kernel would make: an index outside the gap, a score off by 2e-4 relative, a
masked or out-of-range pick, an empty row reported as a pick, a live row
reported empty, and a pick just outside the gap.  (The methodology of a
parity check that must be shown to fail on a perturbed answer follows the
regolith audit "opus_r22_gr", section "parity".)
"""
import numpy as np
import pytest

import oracle
import synth
from parity import REL_GAP, REL_SCORE, check, l2_floor


def _fp32_answer(o_idx, o_val):
    """What a correct fp32 kernel returns: the oracle's index and its value
    rounded to fp32 (NaN for an empty row)."""
    score = np.where(o_idx >= 0, o_val, np.nan).astype(np.float32)
    return o_idx.astype(np.int32).copy(), score


def _dense(metric):
    Q, C = synth.dense_case(64, 300, 24, "unit" if metric in (2, 3) else "normal", key=90 + metric)
    o_idx, o_val, o_gap = oracle.dense(Q, C, metric)
    floor = l2_floor(Q, C, o_idx) if metric in (0, 1) else 1e-2
    pv = lambda r, c: oracle.pair_values(Q, C, metric, r, c)  # noqa: E731
    return Q, C, o_idx, o_val, o_gap, floor, pv


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
def test_correct_answer_passes(metric):
    Q, C, o_idx, o_val, o_gap, floor, pv = _dense(metric)
    idx, score = _fp32_answer(o_idx, o_val)
    fails, stats = check(idx, score, o_idx, o_val, o_gap, metric, floor, pv)
    assert fails == [] and stats["same_index"] == 64 and stats["gap_accepted"] == 0


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
def test_index_outside_gap_fails(metric):
    Q, C, o_idx, o_val, o_gap, floor, pv = _dense(metric)
    idx, score = _fp32_answer(o_idx, o_val)
    r = int(np.argmax(o_gap))  # the widest gap: any other index is outside it
    idx[r] = (idx[r] + 1) % C.shape[0]
    fails, _ = check(idx, score, o_idx, o_val, o_gap, metric, floor, pv)
    assert any("outside the gap" in f for f in fails), fails


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
@pytest.mark.parametrize("sign", [1, -1])
def test_score_off_by_2e4_fails(metric, sign):
    Q, C, o_idx, o_val, o_gap, floor, pv = _dense(metric)
    idx, score = _fp32_answer(o_idx, o_val)
    scale = np.maximum(np.abs(o_val), np.broadcast_to(floor, o_val.shape))
    r = int(np.argmax(np.abs(o_val) >= scale))  # a row where the relative bound applies
    assert abs(o_val[r]) >= scale[r]
    score[r] = np.float32(o_val[r] + sign * 2 * REL_SCORE * abs(o_val[r]))
    fails, _ = check(idx, score, o_idx, o_val, o_gap, metric, floor, pv)
    assert any("scores off" in f for f in fails), fails
    # half the tolerance passes
    score[r] = np.float32(o_val[r] + sign * 0.5 * REL_SCORE * abs(o_val[r]))
    assert check(idx, score, o_idx, o_val, o_gap, metric, floor, pv)[0] == []


def _near_tie_case():
    """d = 1, q = 0: candidate values 4.0 (c0 = 2), 4.0 (c1 = -2, an exact
    duplicate value), 4 (1 + 2^-22) (c2, 4.8e-7 relative above: inside a
    1e-5 gap), 4.004 (c3, outside) and c4 = 2 (masked in the masked case)."""
    Q = np.zeros((1, 1), np.float32)
    C = np.array([[2.0], [-2.0], [np.float32(2.0) * np.float32(1 + 2.0 ** -23)], [2.001],
                  [2.0]], np.float32)
    return Q, C


def test_pick_inside_gap_passes_and_outside_fails():
    Q, C = _near_tie_case()
    Cl = C[[0, 2, 3]]  # no duplicate: best 4.0 (idx 0), second 4(1+2^-22)
    o_idx, o_val, o_gap = oracle.dense(Q, Cl, 0)
    assert o_idx[0] == 0 and 0 < o_gap[0] <= REL_GAP * o_val[0]
    pv = lambda r, c: oracle.pair_values(Q, Cl, 0, r, c)  # noqa: E731
    floor = l2_floor(Q, Cl, o_idx)
    # the second candidate is inside the gap
    fails, stats = check(np.array([1]), np.array([o_val[0]], np.float32), o_idx, o_val, o_gap, 0,
                         floor, pv)
    assert fails == [] and stats["gap_accepted"] == 1
    # the third is not
    fails, _ = check(np.array([2]), np.array([o_val[0]], np.float32), o_idx, o_val, o_gap, 0,
                     floor, pv)
    assert any("outside the gap" in f for f in fails), fails


def test_duplicate_value_in_gap_accepted_by_rule():
    """Two candidates with the same value (gap 0): the rule accepts either
    index; the lowest-index requirement for exact duplicates is a separate,
    direct check in the tests that build duplicates."""
    Q, C = _near_tie_case()
    o_idx, o_val, o_gap = oracle.dense(Q, C[:2], 0)
    assert o_idx[0] == 0 and o_gap[0] == 0.0
    pv = lambda r, c: oracle.pair_values(Q, C[:2], 0, r, c)  # noqa: E731
    fails, stats = check(np.array([1]), np.array([4.0], np.float32), o_idx, o_val, o_gap, 0,
                         l2_floor(Q, C[:2], o_idx), pv)
    assert fails == [] and stats["gap_accepted"] == 1


def test_masked_or_out_of_range_pick_fails():
    """A near-tie row whose GPU pick is a masked candidate, or an index past
    the table, fails through the legality test."""
    Q, C = _near_tie_case()
    mask = np.zeros((1, 1), np.uint32)
    mask[0, 0] = np.uint32(1 << 0)  # only c0 masked
    o_idx, o_val, o_gap = oracle.dense(Q, C, 0, mask=mask)
    assert o_idx[0] == 1 and o_gap[0] == 0.0  # c1 and c4 tie at 4.0

    def legal(r, c):
        ok = (c >= 0) & (c < C.shape[0])
        ok[ok] &= ((mask[r[ok], c[ok] // 32] >> (c[ok] % 32).astype(np.uint32)) & 1) == 0
        return ok

    pv = lambda r, c: oracle.pair_values(Q, C, 0, r, c)  # noqa: E731
    floor = l2_floor(Q, C, o_idx)
    s = np.array([4.0], np.float32)
    # c4: legal, same value -> accepted
    assert check(np.array([4]), s, o_idx, o_val, o_gap, 0, floor, pv, legal)[0] == []
    # c0: same value but masked -> rejected
    fails, _ = check(np.array([0]), s, o_idx, o_val, o_gap, 0, floor, pv, legal)
    assert any("outside the gap" in f for f in fails), fails
    # past the end of the table -> rejected without evaluating it
    fails, _ = check(np.array([5]), s, o_idx, o_val, o_gap, 0, floor, pv, legal)
    assert fails, fails
    # -1 on a live row -> rejected (score NaN also fails the score bound)
    fails, _ = check(np.array([-1]), np.array([np.nan], np.float32), o_idx, o_val, o_gap, 0,
                     floor, pv, legal)
    assert any("scores off" in f for f in fails) and len(fails) >= 2, fails


def test_empty_row_must_report_minus_one_and_nan():
    Q, C = _near_tie_case()
    mask = np.full((2, 1), np.uint32(0x1F), np.uint32)  # every candidate masked
    mask[1, 0] = 0
    o_idx, o_val, o_gap = oracle.dense(np.zeros((2, 1), np.float32), C, 0, mask=mask)
    assert o_idx[0] == -1 and np.isnan(o_val[0]) and o_idx[1] == 0
    pv = lambda r, c: oracle.pair_values(np.zeros((2, 1), np.float32), C, 0, r, c)  # noqa: E731
    floor = 1e-2
    good_idx = np.array([-1, 0], np.int32)
    good_s = np.array([np.nan, 4.0], np.float32)
    assert check(good_idx, good_s, o_idx, o_val, o_gap, 0, floor, pv)[0] == []
    for idx, s in ((np.array([0, 0]), good_s), (np.array([-1, 0]), np.array([4.0, 4.0])),
                   (np.array([3, 0]), np.array([4.0, 4.0]))):
        fails, _ = check(idx.astype(np.int32), s.astype(np.float32), o_idx, o_val, o_gap, 0, floor,
                         pv)
        assert any("empty-set" in f for f in fails), (idx, s, fails)


def test_floor_bound_rows_are_counted():
    """A query equal to a candidate has s* = 0: the scale is the floor there,
    and the stats say on how many rows that happened."""
    Q, C = synth.dense_case(8, 50, 16, "normal", key=5)
    Q[3] = C[7]
    o_idx, o_val, o_gap = oracle.dense(Q, C, 0)
    idx, score = _fp32_answer(o_idx, o_val)
    fails, stats = check(idx, score, o_idx, o_val, o_gap, 0, l2_floor(Q, C, o_idx),
                         lambda r, c: oracle.pair_values(Q, C, 0, r, c))
    assert fails == [] and stats["floor_bound"] == 1


# ---- the parity tests would catch a kernel with a classic mistake ----------
# A kernel that makes one of these mistakes returns what the oracle built
# with the same planted mistake returns; on inputs shaped like the GPU parity
# cases (a ragged last tile, exact duplicates, masks), the acceptance rule
# against the correct oracle must reject that answer.

def _mutant_answer_fails(Q, C, metric, mutant, mask=None):
    o_idx, o_val, o_gap = oracle.dense(Q, C, metric, mask=mask)
    m_idx, m_val, _ = oracle.dense(Q, C, metric, mask=mask, mutant=mutant)
    score = np.where(m_idx >= 0, m_val, np.nan).astype(np.float32)
    floor = l2_floor(Q, C, o_idx) if metric in (0, 1) else 1e-2

    def legal(r, c):
        ok = (c >= 0) & (c < C.shape[0])
        if mask is not None:
            ok[ok] &= ((mask[r[ok], c[ok] // 32] >> (c[ok] % 32).astype(np.uint32)) & 1) == 0
        return ok
    fails, _ = check(m_idx, score, o_idx, o_val, o_gap, metric, floor,
                     lambda r, c: oracle.pair_values(Q, C, metric, r, c), legal)
    return bool(fails)


@pytest.mark.parametrize("mutant,what", [(2, "last candidate dropped"), (3, "MAX ranked as MIN"),
                                         (4, "last coordinate dropped")])
def test_rule_rejects_mutant_kernels(mutant, what):
    # 130 queries x 97 candidates (ragged against 32/64-row tiles), the last
    # candidate planted as the best match of the first query; d = 33
    Q, C = synth.dense_case(130, 97, 33, "normal", key=70 + mutant)
    C[96] = Q[0] * np.float32(1.0001)
    metric = 1 if mutant == 3 else 0
    assert _mutant_answer_fails(Q, C, metric, mutant), what


def test_rule_rejects_highest_index_ties_through_the_duplicate_check():
    """Ties broken toward the highest index pass the gap rule (the values are
    equal) but not the direct lowest-index check of the duplicate tests."""
    Q, C = synth.dense_case(40, 60, 8, "normal", key=77)
    C[50] = C[7]
    Q[3] = C[7] + np.float32(0.01)
    o_idx, _, _ = oracle.dense(Q, C, 0)
    m_idx, _, _ = oracle.dense(Q, C, 0, mutant=1)
    assert o_idx[3] == 7 and m_idx[3] == 50


def test_rule_rejects_an_ignored_mask():
    Q, C = synth.dense_case(50, 90, 12, "normal", key=78)
    mask = synth.random_mask(50, 90, 0.5, key=79)
    assert _mutant_answer_fails(Q, C, 0, 5, mask=mask)
