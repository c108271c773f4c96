"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-enumerated cases under tests/golden/ (plane geometry, cited);
  * independent library routines: scipy.spatial.distance.cdist and
    sklearn's pairwise_distances_argmin (numpy's argmin documents that the
    first occurrence wins, which is the lowest-index tie-break); the values
    of single (query, candidate) pairs, which the parity rule uses to judge
    near-tie picks, against cdist entries and a hand-worked case;
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
from goldens import csr_cases, diversity_centroid, diversity_walk, hand_cases

MUTANTS = list(range(1, 19))


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


def pin_pair_values(m=0):
    """orc_pair_values against scipy's cdist entries: every metric, queries
    and candidates of different counts in both directions, (query, candidate)
    pairs drawn with repeats and in no order, plus a hand-worked case.  Q and
    C are two slices of one buffer long enough that a build which reads rows
    past either slice (indices exchanged, a wrong row stride) stays inside
    memory and fails on the values instead of faulting."""
    bad = []
    rng = np.random.default_rng(1717)
    for metric in range(4):
        for nq, nc, d in ((13, 41, 7), (37, 5, 3), (6, 6, 1), (9, 200, 33)):
            buf = rng.standard_normal((2 * (nq + nc), d)).astype(np.float32)
            Q, C = buf[:nq], buf[nq:nq + nc]
            qi = rng.integers(0, nq, 3 * (nq + nc))
            cj = rng.integers(0, nc, qi.size)
            qi[:4], cj[:4] = [0, 0, nq - 1, nq - 1], [nc - 1, nc - 1, 0, 0]  # repeats, ends
            if metric in (0, 1):
                D = cdist(Q.astype(np.float64), C.astype(np.float64), "sqeuclidean")
            else:
                D = 1.0 - cdist(Q.astype(np.float64), C.astype(np.float64), "cosine")
            got = oracle.pair_values(Q, C, metric, qi, cj, mutant=m)
            if not np.allclose(got, D[qi, cj], rtol=1e-12, atol=1e-12):
                bad.append(f"pair values metric {metric} shape {(nq, nc, d)}")
    # hand case: q0 = (1, 0), q1 = (0, 2); c0 = (3, 4), c1 = (1, 1), c2 = (-2, 0)
    Q = np.array([[1, 0], [0, 2]], np.float32)
    C = np.array([[3, 4], [1, 1], [-2, 0]], np.float32)
    qi = np.array([0, 1, 1, 0, 0])
    cj = np.array([0, 0, 2, 2, 1])
    exp_l2 = [4 + 16, 9 + 4, 4 + 4, 9, 1]
    exp_cos = [3 / 5, 8 / 10, 0.0, -1.0, 1 / math.sqrt(2)]
    for metric, exp in ((0, exp_l2), (1, exp_l2), (2, exp_cos), (3, exp_cos)):
        got = oracle.pair_values(Q, C, metric, qi, cj, mutant=m)
        if not all(_close(g, e, 1e-12, 1e-12) for g, e in zip(got, exp)):
            bad.append(f"pair values hand case metric {metric}: {list(got)}")
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


# ---- SOM batch update and quantisation error --------------------------------
# Pinned against: group means (np.add.at), a single input (closed form), a
# separable Gaussian window from scipy.signal.windows.gaussian correlated over
# the map by scipy.ndimage.correlate (zero outside the map), the global mean
# when the window is the whole map and sigma is huge, mirror/transpose
# symmetry of the map, a hand-worked 1x3 map, and distances with known roots.

def _som_inputs(n, d, nc, key, dense=True):
    rng = np.random.default_rng(key)
    X = rng.normal(size=(n, d)).astype(np.float32)
    if not dense:
        X[rng.random(X.shape) < 0.7] = 0.0
    bmu = rng.integers(0, nc, n).astype(np.int32)
    C = rng.normal(size=(nc, d)).astype(np.float32)
    return X, bmu, C


def _som(X, bmu, C, rows, cols, sigma, R, m=0, **kw):
    ip, ix, v = oracle.dense_as_csr(X)
    return oracle.som_update(ip, ix, v, X.shape[1], bmu, C, rows, cols, sigma, R, mutant=m, **kw)


def _group_sums(X, bmu, nc):
    S = np.zeros((nc, X.shape[1]))
    np.add.at(S, bmu, X.astype(np.float64))
    return S, np.bincount(bmu, minlength=nc).astype(np.float64)


def pin_som_group_mean(m=0):
    bad = []
    rows, cols = 3, 5
    X, bmu, C = _som_inputs(40, 6, rows * cols, key=70)
    bmu[bmu == 7] = 8  # leave neuron 7 without inputs
    S, N = _group_sums(X, bmu, rows * cols)
    ref = np.where(N[:, None] > 0, S / np.maximum(N, 1)[:, None], C)
    for sigma, R in ((1.0, 0), (1e-3, 2)):
        w, _, _ = _som(X, bmu, C, rows, cols, sigma, R, m)
        if not np.allclose(w, ref, rtol=1e-12, atol=1e-12):
            bad.append(f"som: sigma {sigma} R {R} is not the per-neuron mean")
    return bad


def pin_som_single_input(m=0):
    rows, cols, R = 6, 9, 2
    X, _, C = _som_inputs(1, 5, rows * cols, key=71)
    b = 3 * cols + 7  # (3, 7): the window is clipped by the right edge
    w, _, den = _som(X, np.array([b], np.int32), C, rows, cols, 1.3, R, m)
    y, x = np.divmod(np.arange(rows * cols), cols)
    inside = (np.abs(y - 3) <= R) & (np.abs(x - 7) <= R)
    ref = np.where(inside[:, None], X[0].astype(np.float64), C)
    ok = np.allclose(w, ref, rtol=1e-12, atol=1e-12) and np.array_equal(den > 0, inside)
    return [] if ok else ["som: one input must move exactly its window onto itself"]


def pin_som_scipy(m=0):
    from scipy.ndimage import correlate
    from scipy.signal.windows import gaussian
    bad = []
    for rows, cols, sigma, R, key in ((7, 11, 1.5, 3, 72), (10, 4, 0.8, 2, 73), (5, 5, 2.5, 6, 74)):
        nc = rows * cols
        X, bmu, C = _som_inputs(60, 4, nc, key)
        bmu[::7] = 0  # a crowded corner neuron
        S, N = _group_sums(X, bmu, nc)
        g = gaussian(2 * R + 1, std=sigma)
        K = np.outer(g, g)
        den = correlate(N.reshape(rows, cols), K, mode="constant", cval=0.0).reshape(-1)
        num = np.stack([correlate(S[:, k].reshape(rows, cols), K, mode="constant", cval=0.0)
                        .reshape(-1) for k in range(S.shape[1])], axis=1)
        ref = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1)[:, None], C)
        w, mass, d = _som(X, bmu, C, rows, cols, sigma, R, m)
        if not (np.allclose(w, ref, rtol=1e-10, atol=1e-10) and np.allclose(d, den, rtol=1e-12)):
            bad.append(f"som differs from the scipy window on {rows}x{cols} R {R}")
        A, _ = _group_sums(np.abs(X), bmu, nc)
        lin = np.stack([correlate(A[:, k].reshape(rows, cols), K, mode="constant")
                        .reshape(-1) for k in range(A.shape[1])], axis=1)
        ref_mass = np.where(den[:, None] > 0, lin / np.where(den > 0, den, 1)[:, None], 0.0)
        if not np.allclose(mass, ref_mass, rtol=1e-10, atol=1e-12):
            bad.append("som mass is not the smoothed |x|")
    return bad


def pin_som_global_mean(m=0):
    rows, cols = 4, 6
    X, bmu, C = _som_inputs(30, 5, rows * cols, key=75)
    w, _, _ = _som(X, bmu, C, rows, cols, 1e6, max(rows, cols), m)
    ref = X.astype(np.float64).mean(axis=0)
    return [] if np.allclose(w, ref[None, :], rtol=1e-9, atol=1e-9) else ["som: huge window is not the mean"]


def pin_som_symmetry(m=0):
    rows, cols = 4, 7
    X, bmu, C = _som_inputs(50, 3, rows * cols, key=76)
    y, x = np.divmod(np.arange(rows * cols), cols)
    w0, _, _ = _som(X, bmu, C, rows, cols, 1.1, 2, m)
    mir = y * cols + (cols - 1 - x)          # mirror left-right
    w1, _, _ = _som(X, mir[bmu].astype(np.int32), C[np.argsort(mir)], rows, cols, 1.1, 2, m)
    tr = x * rows + y                         # transpose: the map becomes cols x rows
    w2, _, _ = _som(X, tr[bmu].astype(np.int32), C[np.argsort(tr)], cols, rows, 1.1, 2, m)
    bad = []
    if not np.allclose(w1[mir], w0, rtol=1e-12, atol=1e-12):
        bad.append("som not mirror-symmetric")
    if not np.allclose(w2[tr], w0, rtol=1e-12, atol=1e-12):
        bad.append("som not transpose-symmetric")
    return bad


def pin_som_hand(m=0):
    # 1 x 3 map, sigma 1, R 1; x = 1 at neuron 0 and x = 4 at neuron 2.  Neuron 0
    # sees only its own input (neuron 2 is two steps away), neuron 1 sees both
    # with the same weight (midpoint 2.5), neuron 2 only its own.
    X = np.array([[1.0], [4.0]], np.float32)
    w, _, _ = _som(X, np.array([0, 2], np.int32), np.zeros((3, 1), np.float32), 1, 3, 1.0, 1, m)
    return [] if np.allclose(w[:, 0], [1.0, 2.5, 4.0], rtol=0, atol=1e-15) else [f"som hand {w[:, 0]}"]


def pin_som_csr_duplicates(m=0):
    # a column repeated within a row adds its values: [2 + 3] at column 1
    ip = np.array([0, 2, 3], np.int64)
    a = oracle.som_update(ip, np.array([1, 1, 0], np.int32), np.array([2, 3, 7], np.float32), 2,
                          np.array([0, 0], np.int32), np.zeros((1, 2), np.float32), 1, 1, 1.0, 0,
                          mutant=m)[0]
    return [] if np.allclose(a, [[3.5, 2.5]], atol=1e-15) else ["som csr duplicates"]


def pin_qe(m=0):
    bad = []
    # distances 5, 1, 10 from the origin neuron (3-4-5 and 6-8-10 triangles)
    X = np.array([[3, 4], [0, 1], [6, 8]], np.float32)
    C = np.array([[0, 0], [100, 100]], np.float32)
    _, v, _ = oracle.dense(X, C, 0, mutant=m)
    if not _close(oracle.mean_sqrt(v, mutant=m), 16.0 / 3.0, 1e-14, 1e-14):
        bad.append("qe of 5, 1, 10")
    # inputs sitting on neurons have zero error
    _, C2 = synth.dense_case(1, 9, 4, "normal", key=77)
    _, v2, _ = oracle.dense(C2[[3, 5, 3]], C2, 0, mutant=m)
    if oracle.mean_sqrt(v2, mutant=m) != 0.0:
        bad.append("qe of inputs equal to neurons")
    if not math.isnan(oracle.mean_sqrt(np.zeros(0), mutant=m)):
        bad.append("qe of no inputs must be NaN")
    return bad


# ---- centroid-reference diversity -------------------------------------------
# Pinned against: the hand-worked plane walk (tests/golden/diversity_centroid.txt);
# the first step equals the last-pick step (the centroid of one row is that
# row); the replay of the oracle's own run accepts every pick; relabelling
# the table's rows relabels the picks; scaling every row by a positive
# constant changes no pick (cosines are scale-free).

def pin_centroid_walk(m=0):
    w = diversity_centroid()
    picks, vals = oracle.div_run_centroid(w["C"], np.array([w["seed"]]), len(w["picks"]),
                                          mutant=m)
    bad = []
    if list(picks[0]) != w["picks"]:
        bad.append(f"centroid walk picks {list(picks[0])}")
    for v, e in zip(vals[0], w["values"]):
        if not _close(v, e, 1e-6, 1e-6):
            bad.append(f"centroid walk value {v} != {e}")
    return bad


def _div_table(n, d, key):
    _, C = synth.dense_case(1, n, d, "unit", key=key)
    (r,) = synth.rng_children(9000 + key, 1)
    return C, r.choice(n, 6, replace=False).astype(np.int32)


def pin_centroid_first_step(m=0):
    C, seeds = _div_table(90, 12, 80)
    a, va = oracle.div_run_centroid(C, seeds, 1, mutant=m)
    b, vb = oracle.div_run(C, seeds, 1, mutant=m)
    ok = np.array_equal(a, b) and np.allclose(va, vb, rtol=1e-12, atol=1e-12)
    return [] if ok else ["centroid step 1 differs from the last-pick step"]


def pin_centroid_replay(m=0):
    C, seeds = _div_table(70, 9, 81)
    picks, vals = oracle.div_run_centroid(C, seeds, 30, mutant=m)
    rep = oracle.div_replay_centroid(C, seeds, picks, mutant=m)
    ok = (rep["pick_ok"].all() and np.array_equal(rep["bidx"], picks)
          and np.allclose(rep["pick_value"], vals, rtol=1e-12, atol=1e-12))
    bad = [] if ok else ["centroid replay rejects the oracle's own run"]
    seen = [set([s]) | set(p) for s, p in zip(seeds, picks)]
    if any(len(sv) != 31 for sv in seen):
        bad.append("centroid run repeats a pick or the seed")
    return bad


def pin_centroid_relabel_and_scale(m=0):
    C, seeds = _div_table(60, 7, 82)
    picks, _ = oracle.div_run_centroid(C, seeds, 20, mutant=m)
    (r,) = synth.rng_children(9100, 1)
    perm = r.permutation(C.shape[0])            # new row i = old row perm[i]
    inv = np.argsort(perm)
    p2, _ = oracle.div_run_centroid(C[perm], inv[seeds].astype(np.int32), 20, mutant=m)
    p3, _ = oracle.div_run_centroid(C * np.float32(4.0), seeds, 20, mutant=m)
    bad = []
    if not np.array_equal(perm[p2], picks):
        bad.append("centroid run not relabelling-invariant")
    if not np.array_equal(p3, picks):
        bad.append("centroid run depends on the rows' scale")
    return bad


PINS = [pin_hand_cases, pin_csr_cases, pin_walk, pin_library, pin_sklearn, pin_closed_forms,
        pin_pair_values,
        pin_split_invariance, pin_permutation, pin_translation, pin_duplicates,
        pin_csr_vs_dense, pin_replay, pin_gram, pin_sqnorms, pin_som_group_mean,
        pin_som_single_input, pin_som_scipy, pin_som_global_mean, pin_som_symmetry,
        pin_som_hand, pin_som_csr_duplicates, pin_qe, pin_centroid_walk,
        pin_centroid_first_step, pin_centroid_replay, pin_centroid_relabel_and_scale]


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
