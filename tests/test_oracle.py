"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-enumerated cases under tests/golden/ (plane geometry, cited);
  * independent library routines: scipy.spatial.distance.cdist and
    sklearn's pairwise_distances_argmin (numpy's argmin documents that the
    first occurrence wins, which is the lowest-index tie-break);
  * closed forms (a query equal to a candidate, an antipodal unit vector);
  * invariants: split/tiling invariance of the arg-reduction (associativity of
    max, "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
    "Intended Behavior"; ragged last tile, "Risks"), permutation invariance,
    translation invariance of squared L2 on exactly representable data,
    duplicates -> lowest index;
  * the sparse scan against the dense scan on densified rows;
  * the diversity replay against the directly run sequence.
Each pin is a function returning a list of failures so that the non-vacuity
test can run the same pins on oracle builds with one planted mistake.
"""
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import oracle
import synth
from goldens import csr_cases, diversity_walk, hand_cases

MUTANTS = list(range(1, 10))


def _close(a, b, rel=1e-12, abs_=1e-12):
    if math.isnan(b):
        return math.isnan(a)
    return abs(a - b) <= max(abs_, rel * abs(b))


# ------------------------------------------------------------------ pins --

def pin_hand_cases(m=0):
    bad = []
    for c in hand_cases():
        idx, val, gap = oracle.dense(c["Q"], c["C"], c["metric"], mask=c["mask_words"], mutant=m)
        if idx[0] != c["expect_idx"] or not _close(val[0], c["expect_value"], 1e-6, 1e-6):
            bad.append(f"{c['name']}: got ({idx[0]}, {val[0]})")
    return bad


def pin_csr_cases(m=0):
    CT, rows = csr_cases()
    bad = []
    for r in rows:
        indptr = np.array([0, len(r["idx"])], np.int32)
        idx, val, _ = oracle.csr(indptr, np.array(r["idx"], np.int32),
                                 np.array(r["val"], np.float32), CT, r["metric"], mutant=m)
        if idx[0] != r["expect_idx"] or not _close(val[0], r["expect_value"], 1e-6, 1e-6):
            bad.append(f"csr {r}: got ({idx[0]}, {val[0]})")
    return bad


def pin_walk(m=0):
    w = diversity_walk()
    picks, vals = oracle.div_run(w["C"], np.array([w["seed"]]), len(w["picks"]), mutant=m)
    bad = []
    if list(picks[0]) != w["picks"]:
        bad.append(f"walk picks {list(picks[0])}")
    for got, exp in zip(vals[0], w["values"]):
        if not _close(got, exp, 1e-12, 1e-12):
            bad.append(f"walk value {got} vs {exp}")
    return bad


def _lib_argbest(Q, C, metric, mask=None):
    """Library reference: scipy cdist + numpy first-occurrence arg-reduction."""
    if metric in (0, 1):
        D = cdist(Q.astype(np.float64), C.astype(np.float64), "sqeuclidean")
    else:
        D = 1.0 - cdist(Q.astype(np.float64), C.astype(np.float64), "cosine")
    key = D if metric in (0, 3) else -D
    if mask is not None:
        nc = C.shape[0]
        bits = np.unpackbits(mask.view(np.uint8), bitorder="little", axis=1)[:, :nc].astype(bool)
        key = np.where(bits, np.inf, key)
    idx = key.argmin(axis=1)
    return idx, D[np.arange(len(idx)), idx]


def pin_library(m=0):
    bad = []
    for metric in range(4):
        for key, (nq, nc, d) in enumerate([(40, 300, 17), (7, 1000, 3), (25, 64, 64)]):
            Q, C = synth.dense_case(nq, nc, d, "normal", key=key * 10 + metric)
            mask = synth.random_mask(nq, nc, 0.3, key=key) if key == 1 else None
            idx, val, _ = oracle.dense(Q, C, metric, mask=mask, mutant=m)
            li, lv = _lib_argbest(Q, C, metric, mask)
            if not (idx == li).all():
                bad.append(f"library metric {metric} shape {(nq, nc, d)}: idx differs")
            elif not np.allclose(val, lv, rtol=1e-9, atol=1e-9):
                bad.append(f"library metric {metric}: values differ")
    return bad


def pin_sklearn(m=0):
    from sklearn.metrics import pairwise_distances_argmin
    Q, C = synth.dense_case(60, 500, 9, "normal", key=99)
    idx, _, _ = oracle.dense(Q, C, 0, mutant=m)
    ref = pairwise_distances_argmin(Q.astype(np.float64), C.astype(np.float64))
    return [] if (idx == ref).all() else ["sklearn argmin differs"]


def pin_closed_forms(m=0):
    bad = []
    Q, C = synth.dense_case(1, 200, 33, "normal", key=7)
    for j in (0, 57, 199):
        idx, val, gap = oracle.dense(C[j:j + 1], C, 0, mutant=m)
        if idx[0] != j or val[0] != 0.0 or not gap[0] > 0:
            bad.append(f"self-match {j}: ({idx[0]}, {val[0]})")
    _, U = synth.dense_case(1, 150, 12, "unit", key=8)
    for j in (3, 149):
        idx, val, _ = oracle.dense(-U[j:j + 1], U, 3, mutant=m)
        if idx[0] != j or not _close(val[0], -1.0, 1e-6, 1e-6):
            bad.append(f"antipode {j}: ({idx[0]}, {val[0]})")
        idx, val, _ = oracle.dense(U[j:j + 1], U, 2, mutant=m)
        if idx[0] != j or not _close(val[0], 1.0, 1e-6, 1e-6):
            bad.append(f"cos self {j}: ({idx[0]}, {val[0]})")
    return bad


def pin_split_invariance(m=0):
    """Whole-range scan == min over any tiling, ragged last tile included."""
    bad = []
    rng = np.random.default_rng(11)
    for metric in range(4):
        Q, C = synth.dense_case(12, 257, 10, "normal", key=20 + metric)
        whole_i, whole_v, _ = oracle.dense(Q, C, metric, mutant=m)
        for trial in range(4):
            cuts = np.sort(rng.choice(np.arange(1, 257), size=rng.integers(1, 9), replace=False))
            edges = [0, *cuts.tolist(), 257]
            best_k = np.full(12, np.inf)
            best_i = np.full(12, -1)
            best_v = np.full(12, np.nan)
            for lo, hi in zip(edges[:-1], edges[1:]):
                i, v, _ = oracle.dense(Q, C[lo:hi], metric, mutant=m)
                k = v if metric in (0, 3) else -v
                better = k < best_k  # tiles in ascending order: strict < keeps lowest
                best_k = np.where(better, k, best_k)
                best_i = np.where(better, i + lo, best_i)
                best_v = np.where(better, v, best_v)
            if not (best_i == whole_i).all() or not (best_v == whole_v).all():
                bad.append(f"split metric {metric} edges {edges}")
    return bad


def pin_permutation(m=0):
    bad = []
    rng = np.random.default_rng(5)
    for metric in range(4):
        Q, C = synth.dense_case(20, 140, 8, "normal", key=40 + metric)
        i0, v0, _ = oracle.dense(Q, C, metric, mutant=m)
        p = rng.permutation(140)
        i1, v1, _ = oracle.dense(Q, C[p], metric, mutant=m)
        if not (p[i1] == i0).all() or not np.allclose(v0, v1, rtol=1e-12):
            bad.append(f"candidate permutation metric {metric}")
        r = rng.permutation(20)
        i2, v2, _ = oracle.dense(Q[r], C, metric, mutant=m)
        if not (i2 == i0[r]).all():
            bad.append(f"query permutation metric {metric}")
    return bad


def pin_translation(m=0):
    """Squared L2 is unchanged when queries and candidates move together;
    small-integer data keeps every value exact in float32 and float64."""
    bad = []
    Q, C = synth.dense_case(15, 90, 6, "int", key=3)
    t = np.array([3, -5, 7, 0, 1, -2], np.float32)
    for metric in (0, 1):
        i0, v0, _ = oracle.dense(Q, C, metric, mutant=m)
        i1, v1, _ = oracle.dense(Q + t, C + t, metric, mutant=m)
        if not (i0 == i1).all() or not (v0 == v1).all():
            bad.append(f"translation metric {metric}")
    return bad


def pin_duplicates(m=0):
    bad = []
    Q, C = synth.dense_case(10, 50, 5, "normal", key=4)
    C = np.concatenate([C, C, C])  # rows j, j+50, j+100 identical
    for metric in range(4):
        idx, _, gap = oracle.dense(Q, C, metric, mutant=m)
        if not (idx < 50).all():
            bad.append(f"duplicates metric {metric}: {idx}")
        if not (gap == 0).all():
            bad.append(f"duplicates gap metric {metric}")
    return bad


def pin_csr_vs_dense(m=0):
    bad = []
    (r,) = synth.rng_children(123, 1)
    indptr, indices, values = synth.sparse_rows(r, 30, 200, p=0.05)
    lo, hi = int(indptr[2]), int(indptr[3])  # make row 2 empty
    indices = np.concatenate([indices[:lo], indices[hi:]])
    values = np.concatenate([values[:lo], values[hi:]])
    indptr = indptr.copy()
    indptr[3:] -= hi - lo
    CT = synth.uniform01(r, (200, 333))
    synth.normalize_columns(CT)
    Qd = np.zeros((30, 200), np.float32)
    for i in range(30):
        Qd[i, indices[indptr[i]:indptr[i + 1]]] = values[indptr[i]:indptr[i + 1]]
    for metric in range(4):
        if metric in (2, 3):
            nz = indptr[1:] > indptr[:-1]
        else:
            nz = np.ones(30, bool)
        i_s, v_s, _ = oracle.csr(indptr, indices, values, CT, metric, mutant=m)
        i_d, v_d, _ = oracle.dense(Qd, np.ascontiguousarray(CT.T), metric, mutant=m)
        if not (i_s[nz] == i_d[nz]).all() or not np.allclose(v_s[nz], v_d[nz], rtol=1e-9, atol=1e-12):
            bad.append(f"csr vs dense metric {metric}")
    return bad


def pin_replay(m=0):
    bad = []
    _, C = synth.dense_case(1, 40, 3, "unit", key=50)
    seeds = np.array([0, 7, 39], np.int32)
    picks, vals = oracle.div_run(C, seeds, 20, mutant=m)
    G = oracle.gram_cos(C, mutant=m)
    rep = oracle.div_replay(G, seeds, picks, mutant=m)
    if not (rep["pick_ok"] == 1).all():
        bad.append("replay: own picks illegal")
    if not (rep["bidx"] == picks).all():
        bad.append("replay: bidx differs from the direct run")
    if not np.allclose(rep["pick_value"], vals, rtol=1e-12, atol=1e-15):
        bad.append("replay: values differ")
    for s in range(3):
        row = picks[s]
        if len(set(row.tolist())) != len(row) or seeds[s] in row:
            bad.append("replay: picks repeat or include the seed")
    return bad


def pin_gram(m=0):
    _, C = synth.dense_case(1, 60, 7, "normal", key=51)
    G = oracle.gram_cos(C, mutant=m)
    ref = 1.0 - cdist(C.astype(np.float64), C.astype(np.float64), "cosine")
    return [] if np.allclose(G, ref, atol=1e-12) else ["gram differs from scipy cosine"]


def pin_sqnorms(m=0):
    X = synth.dense_case(1, 37, 11, "normal", key=52)[1]
    ref = np.einsum("ij,ij->i", X.astype(np.float64), X.astype(np.float64))
    a = oracle.sqnorms(X, mutant=m)
    b = oracle.sqnorms(np.ascontiguousarray(X.T), feature_major=True, mutant=m)
    return [] if np.allclose(a, ref, rtol=1e-13) and np.allclose(b, ref, rtol=1e-13) else ["sqnorms"]


PINS = [pin_hand_cases, pin_csr_cases, pin_walk, pin_library, pin_sklearn, pin_closed_forms,
        pin_split_invariance, pin_permutation, pin_translation, pin_duplicates,
        pin_csr_vs_dense, pin_replay, pin_gram, pin_sqnorms]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin(0) == []


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant):
    oracle.build(mutant, force=False)
    assert oracle.mutant_id(mutant) == mutant
    caught = [p.__name__ for p in PINS if p(mutant)]
    assert caught, f"mutant {mutant} passes every pin"


def test_threads_do_not_change_results():
    Q, C = synth.dense_case(33, 400, 16, "normal", key=60)
    a = oracle.dense(Q, C, 0, threads=1)
    b = oracle.dense(Q, C, 0, threads=5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
