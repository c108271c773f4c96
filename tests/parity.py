"""Acceptance rule for comparing the HIP path with the oracle.

Rule (floating point decides an index here, so both parts are needed):
  * score: |score_gpu - s*| <= 1e-4 * scale;
  * index: if the oracle's top-two gap > 1e-5 * scale the GPU index must equal
    the oracle's (bit-exact); otherwise the GPU pick must be a legal candidate
    whose exact value lies inside that gap: key(pick) - key(best) <= 1e-5*scale;
  * no candidate left: index -1 and score NaN.
scale = max(|s*|, floor).  The floor only matters when s* is near zero (a
query that equals a candidate), where a relative bound is meaningless: the
expanded form |q|^2 + |c|^2 - 2 q.c loses about eps32 * (|q|^2 + |c|^2) to
cancellation, so the squared-L2 floor is 1e-2 * (|q|^2 + |c*|^2) (score
tolerance 1e-6 * (|q|^2 + |c*|^2)); cosines of unit rows are O(1), floor 1e-2.
The floor keeps the 1e-4 relative bound for every s* above it; at s* = 0
exactly it is tighter than what fp32 guarantees: |q|^2, |c|^2 and q.c are fp32
sums of d products, each within gamma_d = d u / (1 - d u) (u = 2^-24) of its
value in any order, so the worst case is 2 gamma_{d+1} (|q|^2 + |c|^2), and
rows searched against themselves measured up to about 1.1 sqrt(d) u
(|q|^2 + |c|^2), above 1e-6 (|q|^2 + |c|^2) for some rows at d = 256 and 768.
Exact self-matches are therefore checked against the worst-case bound
(``self_match_tol``), not through this rule.
Exact duplicates are additionally required to return the lowest index (the
tests that build duplicates check idx directly).
"""
import numpy as np

REL_SCORE = 1e-4
REL_GAP = 1e-5


U32 = 2.0 ** -24


def self_match_tol(C):
    """fp32 worst case of the expanded form at s* = 0 for rows C searched
    against themselves: 2 gamma_{d+1} (|c|^2 + |c|^2)."""
    C64 = C.astype(np.float64)
    n = C.shape[1] + 1
    gamma = n * U32 / (1.0 - n * U32)
    return 2.0 * gamma * 2.0 * np.einsum("ij,ij->i", C64, C64)


def l2_floor(Q, C, o_idx):
    Q64 = Q.astype(np.float64)
    qn = np.einsum("ij,ij->i", Q64, Q64)
    cb = C[np.maximum(o_idx, 0)].astype(np.float64)
    cn = np.einsum("ij,ij->i", cb, cb)
    return 1e-2 * (qn + cn)


def check(idx_g, score_g, o_idx, o_val, o_gap, metric, floor, pick_values, legal=None):
    """Return (failures list, stats dict).

    pick_values(rows, cand) -> oracle metric values for (query row, candidate)
    legal(rows, cand) -> bool array, candidate allowed (in range, unmasked)
    """
    idx_g = np.asarray(idx_g).astype(np.int64)
    score_g = np.asarray(score_g, np.float64)
    o_idx = np.asarray(o_idx).astype(np.int64)
    fails = []
    none = o_idx < 0
    if none.any():
        bad = none & ((idx_g != -1) | ~np.isnan(score_g))
        if bad.any():
            fails.append(f"{bad.sum()} empty-set rows without (-1, NaN), e.g. row {np.nonzero(bad)[0][0]}")
    live = ~none
    rows = np.nonzero(live)[0]
    s = o_val[rows]
    scale = np.maximum(np.abs(s), np.broadcast_to(floor, o_val.shape)[rows])
    err = np.abs(score_g[rows] - s)
    bad = ~(err <= REL_SCORE * scale)
    if bad.any():
        r = rows[bad][0]
        fails.append(f"{bad.sum()} scores off, e.g. row {r}: gpu {score_g[r]!r} oracle {o_val[r]!r}")
    exact = o_gap[rows] > REL_GAP * scale
    mism = idx_g[rows] != o_idx[rows]
    bad = exact & mism
    if bad.any():
        r = rows[bad][0]
        fails.append(f"{bad.sum()} indices differ outside the gap, e.g. row {r}: gpu {idx_g[r]} "
                     f"oracle {o_idx[r]} gap {o_gap[r]!r}")
    near = rows[~exact & mism]
    n_gap = 0
    if near.size:
        cand = idx_g[near]
        ok = cand >= 0
        if legal is not None:
            ok &= legal(near, np.maximum(cand, 0))
        v = np.full(near.size, np.nan)
        if ok.any():
            v[ok] = pick_values(near[ok], cand[ok])
        mins = metric in (0, 3)
        dk = (v - o_val[near]) if mins else (o_val[near] - v)
        sc = np.maximum(np.abs(o_val[near]), np.broadcast_to(floor, o_val.shape)[near])
        good = ok & (dk <= REL_GAP * sc)
        if not good.all():
            r = near[~good][0]
            fails.append(f"{(~good).sum()} picks outside the gap, e.g. row {r}: gpu {idx_g[r]}")
        n_gap = int(good.sum())
    # rows whose scale is the floor rather than |s*| (the relative bound
    # became an absolute one there)
    floor_bound = int((np.broadcast_to(floor, o_val.shape)[rows] > np.abs(s)).sum())
    stats = dict(rows=int(o_idx.size), same_index=int((~mism).sum()), gap_accepted=n_gap,
                 empty=int(none.sum()), floor_bound=floor_bound)
    return fails, stats
