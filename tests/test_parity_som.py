"""GPU parity of the SOM epoch around the BMU search (through the C ABI).

"From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof", section 3
(workload): each input's BMU is found, then that neuron and its neighbours are
updated; the update is the batch map with a Gaussian neighbourhood in a square
window (the oracle's reading).

Bar, derived from the arithmetic: the GPU sums each neuron's inputs with fp32
atomics (at most c terms, c = the largest number of inputs sharing a BMU), then
runs two window passes of at most 2R+1 fp32 fused multiply-adds each over the
same magnitudes (the one-sweep kernels add the two taps at +-t first and then
fuse the multiply-add, which puts no more roundings on any term), the same for
the denominator, and multiplies by the
denominator's fp32 reciprocal (two roundings).  Every step adds at
most a unit roundoff u = 2^-24 per term on sum_i h |x_i| / den (the oracle's
``mass``), so |w_gpu - w| <= 2 (c + 8R + 12) u mass (factor 2 for second-order
terms).  Neurons with a zero denominator must keep their weights bit for bit.
The quantisation error is checked against the oracle's mean Euclidean
distance within the bound that the score tolerance of the search implies
(sqrt is monotone: |sqrt(a) - sqrt(s)| <= max(sqrt(s + e) - sqrt(s),
sqrt(s) - sqrt(max(s - e, 0))) for |a - s| <= e).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from parity import REL_SCORE, check, l2_floor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import farthest_vector_search_amd as vs  # noqa: E402

U = 2.0 ** -24


def dev():
    return torch.device("cuda:0")


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def r_eff(R, rows, cols):
    return min(R, max(rows, cols) - 1)


def som_tol(mass, bmu, nc, R):
    b = bmu[(bmu >= 0) & (bmu < nc)]
    c = int(np.bincount(b, minlength=nc).max()) if b.size else 0
    return 2.0 * (c + 8 * R + 12) * U * mass + 1e-37


def check_update(w_gpu, old, w_o, mass, den, bmu, rows, cols, R):
    """w_gpu / old: the requested neurons' rows after / before the update."""
    nc = rows * cols
    tol = som_tol(mass, bmu, nc, r_eff(R, rows, cols))
    keep = den == 0
    bad = []
    if keep.any() and not np.array_equal(w_gpu[keep].view(np.uint32), old[keep].view(np.uint32)):
        bad.append(f"{int((w_gpu[keep] != old[keep]).any(axis=1).sum())} neurons without "
                   "inputs in their window changed")
    live = ~keep
    err = np.abs(w_gpu[live].astype(np.float64) - w_o[live])
    over = err > tol[live]
    if over.any():
        i, k = np.argwhere(over)[0]
        bad.append(f"{int(over.sum())} weights off, e.g. gpu {w_gpu[live][i, k]!r} oracle "
                   f"{w_o[live][i, k]!r} tol {tol[live][i, k]!r}")
    return bad


def unblock(CB, nc, d):
    nb = (nc + 63) // 64
    return CB.reshape(nb, d, 64).transpose(0, 2, 1).reshape(nb * 64, d)[:nc]


def dense_inputs(n, rows, cols, d, key):
    X, C = synth.dense_case(n, rows * cols, d, "normal", key=key)
    return X, C


# ------------------------------------------------------------- update only --

UPDATE_CASES = [
    # rows, cols, d, n, sigma, R
    (32, 32, 64, 256, 1.5, 4),        # the 32 x 32 map of the small BMU workload
    (7, 13, 33, 500, 0.75, 1),        # ragged d, non-square map
    (5, 9, 8, 300, 2.0, 16),          # window larger than the map
    (1, 50, 5, 100, 1.0, 3),          # one-row map
    (40, 1, 7, 80, 1.0, 2),           # one-column map
    (3, 4, 4, 50, 1.0, 0),            # R = 0: per-neuron means
    (16, 16, 256, 2000, 3.0, 9),
    (1, 1, 3, 10, 1.0, 0),            # one neuron
    (37, 45, 70, 3000, 2.0, 6),       # 5 row bands (the last 5 rows), a partial strip,
                                      # waves past the map's columns, a partial feature chunk
]


# "sweep" forces the one-sweep kernel (radii 1..8) on maps too small for it to
# be chosen, "passes" the two-pass kernels; "auto" is the library's choice
@pytest.mark.parametrize("smooth", ["auto", "sweep", "passes"])
@pytest.mark.parametrize("rows,cols,d,n,sigma,R", UPDATE_CASES)
def test_som_update_dense(rows, cols, d, n, sigma, R, smooth, monkeypatch):
    if smooth == "auto":
        monkeypatch.delenv("VS_SOM_SMOOTH", raising=False)
    else:
        monkeypatch.setenv("VS_SOM_SMOOTH", smooth)
    nc = rows * cols
    X, C = dense_inputs(n, rows, cols, d, key=900 + rows * 31 + cols)
    bmu = synth.random_indices(n, nc, key=rows * 100 + cols)
    if n > 20:
        bmu[:5] = -1          # no BMU: pulls nothing
        bmu[5:8] = nc         # out of range: pulls nothing
        bmu[8:20] = nc // 2   # a crowded neuron
    Cg = T(C)
    vs.vs_som_update(T(X), T(bmu), Cg, (rows, cols), sigma, R)
    w_gpu = Cg.cpu().numpy()
    ip, ix, vv = oracle.dense_as_csr(X)
    w_o, mass, den = oracle.som_update(ip, ix, vv, d, bmu, C, rows, cols, float(np.float32(sigma)),
                                       R, threads=8)
    bad = check_update(w_gpu, C, w_o, mass, den, bmu, rows, cols, R)
    assert not bad, bad


def test_som_update_no_inputs_in_window_keeps_codebook():
    rows, cols, d = 9, 9, 6
    X, C = dense_inputs(3, rows, cols, d, key=950)
    bmu = np.array([0, 0, 1], np.int32)  # only the top-left corner moves
    Cg = T(C)
    vs.vs_som_update(T(X), T(bmu), Cg, (rows, cols), 1.0, 2)
    w = Cg.cpu().numpy()
    y, x = np.divmod(np.arange(rows * cols), cols)
    far = (y > 2) | (x > 3)
    assert np.array_equal(w[far].view(np.uint32), C[far].view(np.uint32))
    assert not np.array_equal(w[0], C[0])


# R 1..8 runs the one-sweep kernel (every radius once, with maps narrower and
# wider than its 64-column strips, fewer rows than R, one row, one column);
# R 0 and R > 8 run the two-pass kernels
@pytest.mark.parametrize("rows,cols,d,n,sigma,R,density", [
    (8, 8, 300, 200, 1.5, 3, 0.05),
    (5, 27, 129, 400, 1.0, 2, 0.1),    # nc not a multiple of 64, ragged d
    (9, 64, 16, 200, 0.5, 1, 0.2),
    (12, 200, 24, 500, 1.0, 7, 0.1),   # four strips, the last one partial
    (3, 130, 20, 300, 1.0, 8, 0.1),    # fewer rows than R
    (1, 70, 40, 100, 1.0, 4, 0.2),     # one row
    (70, 1, 40, 100, 2.0, 5, 0.2),     # one column
    (4, 5, 9, 30, 1.0, 6, 0.3),        # window beyond both edges
    (16, 16, 64, 900, 2.0, 16, 0.2),
    (3, 3, 17, 40, 1.0, 0, 0.3),
    # widths a multiple of 64 (row pointers advanced per step)
    (10, 128, 20, 300, 1.0, 5, 0.1),   # two strips
    (70, 64, 8, 400, 2.0, 8, 0.2),     # one strip, many rows
    (5, 192, 33, 200, 1.0, 3, 0.1),    # three strips
    (1, 64, 7, 50, 1.0, 2, 0.3),       # one row
    (2, 128, 5, 40, 1.0, 6, 0.3),      # fewer rows than R
])
def test_som_update_csr(rows, cols, d, n, sigma, R, density):
    nc = rows * cols
    (r,) = synth.rng_children(960 + nc + d, 1)
    indptr, indices, values = synth.sparse_rows(r, n, d, density)
    CT = synth.uniform01(r, (d, nc))
    bmu = synth.random_indices(n, nc, key=970 + nc)
    bmu[:4] = -1
    CB = vs.vs_csr_block_codebook(T(CT))
    vs.vs_som_update_csr(T(indptr), T(indices), T(values), T(bmu), CB, (rows, cols), d, sigma, R)
    w_gpu = unblock(CB.cpu().numpy(), nc, d)
    C_old = np.ascontiguousarray(CT.T)
    w_o, mass, den = oracle.som_update(indptr, indices, values, d, bmu, C_old, rows, cols,
                                       float(np.float32(sigma)), R, threads=8)
    bad = check_update(w_gpu, C_old, w_o, mass, den, bmu, rows, cols, R)
    assert not bad, bad
    # the padding neurons of the last block stay zero
    tail = CB.cpu().numpy().reshape(-1, d, 64)[-1][:, nc % 64:] if nc % 64 else np.zeros(1)
    assert not tail.any()


def test_som_update_csr_bad_spans_pull_nothing():
    """Rows whose indptr span is not inside [0, nnz] (lo < 0, hi < lo,
    hi > nnz) pull nothing even with a valid BMU, and nothing outside the
    CSR arrays is read; the other rows update as usual (the oracle sees the
    bad rows with no BMU)."""
    rows, cols, d, n = 6, 7, 20, 60
    nc = rows * cols
    (r,) = synth.rng_children(985, 1)
    indptr, indices, values = synth.sparse_rows(r, n, d, 0.2)
    nnz = int(indices.shape[0])
    CT = synth.uniform01(r, (d, nc))
    bmu = synth.random_indices(n, nc, key=986)
    indptr = indptr.copy()
    indptr[0] = -3                    # row 0: lo < 0
    indptr[11] = indptr[10] - 1       # row 10: hi < lo (row 11 keeps a valid span)
    indptr[n] = nnz + 50              # row n - 1: hi > nnz
    bad = np.array([0, 10, n - 1])
    bmu[bad] = 5                      # valid BMUs: they would pull neuron 5's window
    CB = vs.vs_csr_block_codebook(T(CT))
    vs.vs_som_update_csr(T(indptr), T(indices), T(values), T(bmu), CB, (rows, cols), d, 1.0, 2)
    w_gpu = unblock(CB.cpu().numpy(), nc, d)
    C_old = np.ascontiguousarray(CT.T)
    o_bmu = bmu.copy()
    o_bmu[bad] = -1
    w_o, mass, den = oracle.som_update(indptr, indices, values, d, o_bmu, C_old, rows, cols,
                                       1.0, 2, threads=8)
    assert not check_update(w_gpu, C_old, w_o, mass, den, o_bmu, rows, cols, 2)


# ------------------------------------------------------ quantisation error --

@pytest.mark.parametrize("n", [0, 1, 2, 1023, 1024, 1025, 65536])
def test_som_qe(n):
    (r,) = synth.rng_children(980 + n, 1)
    s = (r.random(n) * 50.0).astype(np.float32)
    if n > 3:
        s[0] = 0.0
        s[1] = -1e-6   # cancellation can leave a tiny negative squared distance
    q = vs.vs_som_qe(T(s)).cpu().numpy()[0]
    ref = oracle.mean_sqrt(s.astype(np.float64))
    if n == 0:
        assert math.isnan(q)
    else:
        assert abs(q - ref) <= 1e-12 * max(abs(ref), 1e-300)


# ------------------------------------------------------------------ epochs --

def qe_bound(o_val, floor):
    e = REL_SCORE * np.maximum(np.abs(o_val), floor)
    s = np.maximum(o_val, 0.0)
    up = np.sqrt(s + e) - np.sqrt(s)
    down = np.sqrt(s) - np.sqrt(np.maximum(s - e, 0.0))
    return float(np.maximum(up, down).mean())


def clean_neurons(g_bmu, o_bmu, rows, cols, R):
    """Neurons whose window holds neither BMU of any input on which the GPU
    and the oracle disagree (a pick inside the oracle's top-two gap)."""
    nc = rows * cols
    ok = np.ones(nc, bool)
    y, x = np.divmod(np.arange(nc), cols)
    for i in np.nonzero(g_bmu != o_bmu)[0]:
        for b in (g_bmu[i], o_bmu[i]):
            if 0 <= b < nc:
                by, bx = divmod(int(b), cols)
                ok &= ~((np.abs(y - by) <= R) & (np.abs(x - bx) <= R))
    return np.nonzero(ok)[0]


@pytest.mark.parametrize("rows,cols,d,n,sigma,R", [
    (16, 16, 64, 512, 1.5, 4),
    (6, 11, 37, 300, 1.0, 3),
    (4, 4, 8, 1, 1.0, 1),
])
def test_som_epoch_dense(rows, cols, d, n, sigma, R):
    nc = rows * cols
    X, C = dense_inputs(n, rows, cols, d, key=990 + nc)
    Cg = T(C)
    bmu, score, qe = vs.vs_som_epoch(T(X), Cg, (rows, cols), sigma, R)
    torch.cuda.synchronize()
    g_bmu, g_score, g_qe = bmu.cpu().numpy(), score.cpu().numpy(), qe.cpu().numpy()[0]
    w_gpu = Cg.cpu().numpy()
    o_idx, o_val, o_gap = oracle.dense(X, C, 0, threads=8)
    floor = l2_floor(X, C, o_idx)
    fails, _ = check(g_bmu, g_score, o_idx, o_val, o_gap, 0, floor,
                     lambda r, c: oracle.pair_values(X, C, 0, r, c))
    assert not fails, fails
    assert abs(g_qe - oracle.mean_sqrt(o_val)) <= qe_bound(o_val, floor) + 1e-12
    ip, ix, vv = oracle.dense_as_csr(X)
    sel = clean_neurons(g_bmu, o_idx, rows, cols, R)
    assert sel.size >= nc // 2
    w_o, mass, den = oracle.som_update(ip, ix, vv, d, o_idx, C, rows, cols,
                                       float(np.float32(sigma)), R, neurons=sel, threads=8)
    bad = check_update(w_gpu[sel], C[sel], w_o, mass, den, o_idx, rows, cols, R)
    assert not bad, bad


# dense enough that no row is empty: an empty row is equally far from every
# unit-norm neuron, a tie the GPU may break anywhere inside the oracle's gap
@pytest.mark.parametrize("rows,cols,d,n,sigma,R,density", [
    (8, 16, 200, 300, 1.5, 4, 0.05),
    (5, 13, 77, 150, 1.0, 2, 0.25),
])
def test_som_epoch_csr(rows, cols, d, n, sigma, R, density):
    nc = rows * cols
    (r,) = synth.rng_children(1200 + nc, 1)
    indptr, indices, values = synth.sparse_rows(r, n, d, density)
    assert (np.diff(indptr) > 0).all()
    CT = synth.uniform01(r, (d, nc))
    synth.normalize_columns(CT)
    CB = vs.vs_csr_block_codebook(T(CT))
    bmu, score, qe = vs.vs_som_epoch_csr(T(indptr), T(indices), T(values), CB, (rows, cols), d,
                                         sigma, R)
    torch.cuda.synchronize()
    g_bmu, g_score, g_qe = bmu.cpu().numpy(), score.cpu().numpy(), qe.cpu().numpy()[0]
    w_gpu = unblock(CB.cpu().numpy(), nc, d)
    C_old = np.ascontiguousarray(CT.T)
    o_idx, o_val, o_gap = oracle.csr(indptr, indices, values, CT, 0, threads=8)
    Xd = np.zeros((n, d), np.float32)
    for i in range(n):
        Xd[i, indices[indptr[i]:indptr[i + 1]]] = values[indptr[i]:indptr[i + 1]]
    floor = l2_floor(Xd, C_old, o_idx)
    fails, _ = check(g_bmu, g_score, o_idx, o_val, o_gap, 0, floor,
                     lambda r_, c: oracle.pair_values(Xd, C_old, 0, r_, c))
    assert not fails, fails
    assert abs(g_qe - oracle.mean_sqrt(o_val)) <= qe_bound(o_val, floor) + 1e-12
    sel = clean_neurons(g_bmu, o_idx, rows, cols, R)
    assert sel.size >= nc // 2
    w_o, mass, den = oracle.som_update(indptr, indices, values, d, o_idx, C_old, rows, cols,
                                       float(np.float32(sigma)), R, neurons=sel, threads=8)
    bad = check_update(w_gpu[sel], C_old[sel], w_o, mass, den, o_idx, rows, cols, R)
    assert not bad, bad


@pytest.mark.parametrize("rows,cols,d,n,sigma,R,density", [
    (8, 16, 200, 300, 1.5, 4, 0.05),
    (5, 27, 77, 150, 1.0, 2, 0.25),
])
def test_som_epoch_csr_f16(rows, cols, d, n, sigma, R, density):
    """The epoch searching an fp16 copy: BMUs and the error are those of the
    fp16-rounded codebook (checked against the oracle on the rounded
    codebook); the update applies to the fp32 weights (checked against the
    oracle's update of the fp32 codebook with the oracle's BMUs)."""
    nc = rows * cols
    (r,) = synth.rng_children(1300 + nc, 1)
    indptr, indices, values = synth.sparse_rows(r, n, d, density)
    assert (np.diff(indptr) > 0).all()
    CT = synth.uniform01(r, (d, nc))
    synth.normalize_columns(CT)
    CB = vs.vs_csr_block_codebook(T(CT))
    bmu, score, qe = vs.vs_som_epoch_csr_f16(T(indptr), T(indices), T(values), CB, (rows, cols),
                                             d, sigma, R)
    torch.cuda.synchronize()
    g_bmu, g_score, g_qe = bmu.cpu().numpy(), score.cpu().numpy(), qe.cpu().numpy()[0]
    w_gpu = unblock(CB.cpu().numpy(), nc, d)
    C_old = np.ascontiguousarray(CT.T)
    CT16 = CT.astype(np.float16).astype(np.float32)  # the rounded codebook, exact in fp32
    C16 = np.ascontiguousarray(CT16.T)
    o_idx, o_val, o_gap = oracle.csr(indptr, indices, values, CT16, 0, threads=8)
    Xd = np.zeros((n, d), np.float32)
    for i in range(n):
        Xd[i, indices[indptr[i]:indptr[i + 1]]] = values[indptr[i]:indptr[i + 1]]
    floor = l2_floor(Xd, C16, o_idx)
    fails, _ = check(g_bmu, g_score, o_idx, o_val, o_gap, 0, floor,
                     lambda r_, c: oracle.pair_values(Xd, C16, 0, r_, c))
    assert not fails, fails
    assert abs(g_qe - oracle.mean_sqrt(o_val)) <= qe_bound(o_val, floor) + 1e-12
    sel = clean_neurons(g_bmu, o_idx, rows, cols, R)
    assert sel.size >= nc // 2
    w_o, mass, den = oracle.som_update(indptr, indices, values, d, o_idx, C_old, rows, cols,
                                       float(np.float32(sigma)), R, neurons=sel, threads=8)
    bad = check_update(w_gpu[sel], C_old[sel], w_o, mass, den, o_idx, rows, cols, R)
    assert not bad, bad


def test_som_epoch_no_inputs():
    rows, cols, d = 4, 4, 8
    _, C = dense_inputs(1, rows, cols, d, key=1300)
    Cg = T(C)
    X = torch.empty((0, d), dtype=torch.float32, device=dev())
    bmu, score, qe = vs.vs_som_epoch(X, Cg, (rows, cols), 1.0, 2)
    torch.cuda.synchronize()
    assert math.isnan(qe.cpu().numpy()[0])
    assert np.array_equal(Cg.cpu().numpy(), C)


# --------------------------------------------------------- full-size runs --

SOM_SIGMA, SOM_R = 2.0, 6   # the epoch the benchmark times (window radius 3 sigma)


@pytest.mark.slow
def test_workload_2_som_update_sampled():
    """The 128 x 128 map of the dense workload (65,536 inputs, d = 256) at
    full size, in the benchmark's launch configuration; a seeded BMU
    assignment; 256 seeded neurons checked against the oracle."""
    w = synth.workload(2)
    rows = cols = 128
    bmu = synth.random_indices(w["nq"], w["nc"], key=2)
    Cg = T(w["C"])
    vs.vs_som_update(T(w["Q"]), T(bmu), Cg, (rows, cols), SOM_SIGMA, SOM_R)
    sel = synth.sample_queries(w["nc"], 256, key=21)
    w_gpu = Cg.cpu().numpy()[sel]
    ip, ix, vv = oracle.dense_as_csr(w["Q"])
    w_o, mass, den = oracle.som_update(ip, ix, vv, w["d"], bmu, w["C"], rows, cols, SOM_SIGMA,
                                       SOM_R, neurons=sel.astype(np.int32), threads=16)
    bad = check_update(w_gpu, w["C"][sel], w_o, mass, den, bmu, rows, cols, SOM_R)
    assert not bad, bad


@pytest.mark.slow
def test_workload_2_som_epoch():
    """A full epoch on the 128 x 128 map: every BMU against the oracle (all
    65,536 inputs), the quantisation error, and 256 seeded neurons of the
    update computed by the oracle from its own BMUs."""
    w = synth.workload(2)
    rows = cols = 128
    X, C = w["Q"], w["C"]
    Cg = T(C)
    bmu, score, qe = vs.vs_som_epoch(T(X), Cg, (rows, cols), SOM_SIGMA, SOM_R)
    torch.cuda.synchronize()
    g_bmu, g_score, g_qe = bmu.cpu().numpy(), score.cpu().numpy(), qe.cpu().numpy()[0]
    o_idx, o_val, o_gap = oracle.dense(X, C, 0, threads=16)
    floor = l2_floor(X, C, o_idx)
    fails, _ = check(g_bmu, g_score, o_idx, o_val, o_gap, 0, floor,
                     lambda r, c: oracle.pair_values(X, C, 0, r, c))
    assert not fails, fails
    assert abs(g_qe - oracle.mean_sqrt(o_val)) <= qe_bound(o_val, floor) + 1e-12
    clean = clean_neurons(g_bmu, o_idx, rows, cols, SOM_R)
    sel = np.intersect1d(synth.sample_queries(w["nc"], 256, key=22), clean).astype(np.int32)
    assert sel.size >= 200
    ip, ix, vv = oracle.dense_as_csr(X)
    w_o, mass, den = oracle.som_update(ip, ix, vv, w["d"], o_idx, C, rows, cols, SOM_SIGMA,
                                       SOM_R, neurons=sel, threads=16)
    bad = check_update(Cg.cpu().numpy()[sel], C[sel], w_o, mass, den, o_idx, rows, cols, SOM_R)
    assert not bad, bad


@pytest.mark.slow
def test_workload_5_som_update_sampled():
    """The largest map, 512 x 512 (262,144 neurons, d = 256), updated from the
    65,536 inputs of the large dense workload with a seeded BMU assignment;
    256 seeded neurons checked against the oracle."""
    w = synth.workload(5)
    rows = cols = 512
    bmu = synth.random_indices(w["nq"], w["nc"], key=5)
    Cg = T(w["C"])
    vs.vs_som_update(T(w["Q"]), T(bmu), Cg, (rows, cols), SOM_SIGMA, SOM_R)
    sel = synth.sample_queries(w["nc"], 256, key=51)
    w_gpu = Cg.cpu().numpy()[sel]
    ip, ix, vv = oracle.dense_as_csr(w["Q"])
    w_o, mass, den = oracle.som_update(ip, ix, vv, w["d"], bmu, w["C"], rows, cols, SOM_SIGMA,
                                       SOM_R, neurons=sel.astype(np.int32), threads=16)
    bad = check_update(w_gpu, w["C"][sel], w_o, mass, den, bmu, rows, cols, SOM_R)
    assert not bad, bad


@pytest.mark.slow
def test_workload_4_som_update_sampled():
    """The 256 x 256 map of the sparse workload (32,768 CSR rows, d = 16,384)
    at full size over the blocked codebook; a seeded BMU assignment; 48
    seeded neurons checked against the oracle."""
    w = synth.workload(4)
    rows = cols = 256
    d, nc = w["d"], w["nc"]
    bmu = synth.random_indices(w["nq"], nc, key=4)
    CB = vs.vs_csr_block_codebook(T(w["CT"]))
    vs.vs_som_update_csr(T(w["indptr"]), T(w["indices"]), T(w["values"]), T(bmu), CB,
                         (rows, cols), d, SOM_SIGMA, SOM_R)
    sel = synth.sample_queries(nc, 48, key=41).astype(np.int32)
    blk = CB.view(-1, d, 64)
    w_gpu = np.stack([blk[int(m) // 64, :, int(m) % 64].cpu().numpy() for m in sel])
    del CB, blk
    old = np.ascontiguousarray(w["CT"][:, sel].T)
    w_o, mass, den = oracle.som_update(w["indptr"], w["indices"], w["values"], d, bmu, None,
                                       rows, cols, SOM_SIGMA, SOM_R, neurons=sel, threads=16,
                                       old_rows=old)
    bad = check_update(w_gpu, old, w_o, mass, den, bmu, rows, cols, SOM_R)
    assert not bad, bad
