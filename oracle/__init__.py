"""CPU fp64 oracle for the masked arg-reduction scan (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
package ``farthest_vector_search_amd`` never does, and this package never
imports it.  The arithmetic lives in ``oracle.c`` (plain C, double precision,
one query at a time); this module only builds it with gcc, marshals numpy
arrays, and splits independent queries over threads.  Each C call is the
single-threaded scan; threads only run disjoint shards of queries (ctypes
releases the GIL during the call), which changes no result.

Metric codes: 0 squared-L2 min, 1 squared-L2 max, 2 cosine max, 3 cosine min.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")

L2SQ_MIN, L2SQ_MAX, COS_MAX, COS_MIN = 0, 1, 2, 3

_libs: dict[int, ctypes.CDLL] = {}


# ORACLE_SANITIZE=1 loads the AddressSanitizer + UndefinedBehaviorSanitizer
# build instead of the plain one (the process must preload gcc's libasan;
# see tests/test_oracle_sanitized.py)
SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def lib_path(mutant: int = 0, sanitize: bool = False) -> str:
    name = "liboracle" + (f"_m{mutant}" if mutant else "") + ("_san" if sanitize else "") + ".so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc.  ``mutant`` > 0 plants the numbered mistake;
    ``sanitize`` builds it with AddressSanitizer and UndefinedBehaviorSanitizer
    (bounds, use-after-free, signed overflow, misaligned access, ...)."""
    out = lib_path(mutant, sanitize)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           *(SAN_FLAGS if sanitize else []), f"-DORC_MUTANT={int(mutant)}", _SRC, "-o", tmp,
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load(mutant: int = 0) -> ctypes.CDLL:
    if mutant in _libs:
        return _libs[mutant]
    path = build(mutant, force=False, sanitize=SANITIZE)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    INT = ctypes.c_int
    lib.orc_dense.argtypes = [P, P, I64, I64, I64, INT, P, P, P, P]
    lib.orc_pair_values.argtypes = [P, P, I64, INT, I64, P, P, P]
    lib.orc_sqnorms.argtypes = [P, I64, I64, INT, P]
    lib.orc_csr.argtypes = [P, P, P, I64, P, I64, I64, INT, P, P, P, P, P]
    lib.orc_div_run.argtypes = [P, I64, I64, I64, INT, P, P, P, P]
    lib.orc_gram_cos.argtypes = [P, I64, I64, I64, I64, P]
    lib.orc_div_replay.argtypes = [P, I64, I64, INT, P, P, P, P, P, P, P, P]
    lib.orc_som_update.argtypes = [P, P, P, I64, INT, P, INT, INT, ctypes.c_double, INT, P,
                                   I64, P, P, P, P]
    lib.orc_mean_sqrt.argtypes = [P, I64]
    lib.orc_mean_sqrt.restype = ctypes.c_double
    lib.orc_div_run_centroid.argtypes = [P, I64, I64, I64, INT, P, P, P, P, P]
    lib.orc_div_replay_centroid.argtypes = [P, I64, I64, I64, INT, P, P, P, P, P, P, P, P, P]
    lib.orc_div_run_centroid.restype = None
    lib.orc_div_replay_centroid.restype = None
    lib.orc_mutant.restype = INT
    for f in (lib.orc_dense, lib.orc_pair_values, lib.orc_sqnorms, lib.orc_csr,
              lib.orc_div_run, lib.orc_gram_cos, lib.orc_div_replay, lib.orc_som_update):
        f.restype = None
    _libs[mutant] = lib
    return lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _shards(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    edges = [n * i // parts for i in range(parts + 1)]
    return [(edges[i], edges[i + 1]) for i in range(parts) if edges[i + 1] > edges[i]]


def dense(Q, C, metric: int, mask=None, threads: int = 1, mutant: int = 0):
    """Exact scan of every query row of Q against every row of C.

    Returns (idx int32[nq], value float64[nq], gap float64[nq]).  ``mask`` is
    an optional uint32 array [nq, ceil(nc/32)] (bit set = excluded).
    """
    lib = _load(mutant)
    Q = _c(Q, np.float32)
    C = _c(C, np.float32)
    nq, d = Q.shape
    nc = C.shape[0]
    assert C.shape[1] == d
    W = (nc + 31) // 32
    if mask is not None:
        mask = _c(mask, np.uint32)
        assert mask.shape == (nq, W)
    idx = np.empty(nq, np.int32)
    val = np.empty(nq, np.float64)
    gap = np.empty(nq, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        lib.orc_dense(_p(Q[lo:hi]), _p(C), hi - lo, nc, d, metric,
                      None if mask is None else _p(mask[lo:hi]),
                      _p(idx[lo:hi]), _p(val[lo:hi]), _p(gap[lo:hi]))

    shards = _shards(nq, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return idx, val, gap


def pair_values(Q, C, metric: int, qi, cj, mutant: int = 0):
    """Metric value of the pairs (Q[qi[p]], C[cj[p]])."""
    lib = _load(mutant)
    Q = _c(Q, np.float32)
    C = _c(C, np.float32)
    qi = _c(qi, np.int64)
    cj = _c(cj, np.int64)
    assert qi.shape == cj.shape
    assert (qi >= 0).all() and (qi < Q.shape[0]).all()
    assert (cj >= 0).all() and (cj < C.shape[0]).all()
    out = np.empty(qi.shape[0], np.float64)
    lib.orc_pair_values(_p(Q), _p(C), Q.shape[1], metric, qi.shape[0], _p(qi), _p(cj), _p(out))
    return out


def sqnorms(X, feature_major: bool = False, threads: int = 1, mutant: int = 0):
    """Squared norms (double) of the rows of X, or of its columns when
    ``feature_major`` (X is d x n, one column per candidate)."""
    lib = _load(mutant)
    X = _c(X, np.float32)
    if feature_major:
        d, n = X.shape
    else:
        n, d = X.shape
    out = np.empty(n, np.float64)
    if not feature_major:
        def run(lo_hi):
            lo, hi = lo_hi
            lib.orc_sqnorms(_p(X[lo:hi]), hi - lo, d, 0, _p(out[lo:hi]))
    else:
        # a column block of a feature-major matrix is not contiguous: copy it
        def run(lo_hi):
            lo, hi = lo_hi
            blk = np.ascontiguousarray(X[:, lo:hi])
            tmp = np.empty(hi - lo, np.float64)
            lib.orc_sqnorms(_p(blk), hi - lo, d, 1, _p(tmp))
            out[lo:hi] = tmp
    shards = _shards(n, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return out


def csr(indptr, indices, values, CT, metric: int, col_sq=None, threads: int = 1,
        mutant: int = 0):
    """Exact scan of CSR query rows against the feature-major codebook CT
    (d x nc).  Returns (idx, value, gap) like :func:`dense`."""
    lib = _load(mutant)
    indptr = _c(indptr, np.int32)
    indices = _c(indices, np.int32)
    values = _c(values, np.float32)
    CT = _c(CT, np.float32)
    d, nc = CT.shape
    nq = indptr.shape[0] - 1
    if col_sq is None:
        col_sq = sqnorms(CT, feature_major=True, threads=threads, mutant=mutant)
    col_sq = _c(col_sq, np.float64)
    idx = np.empty(nq, np.int32)
    val = np.empty(nq, np.float64)
    gap = np.empty(nq, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        acc = np.empty(nc, np.float64)
        sub_ptr = np.ascontiguousarray(indptr[lo:hi + 1])  # absolute offsets kept
        lib.orc_csr(_p(sub_ptr), _p(indices), _p(values), hi - lo, _p(CT), nc, d, metric,
                    _p(col_sq), _p(acc), _p(idx[lo:hi]), _p(val[lo:hi]), _p(gap[lo:hi]))

    shards = _shards(nq, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return idx, val, gap


def div_run(C, seeds, T: int, mutant: int = 0):
    """Greedy diversity sequences computed directly.  Returns (picks, cosines),
    both [nseq, T]; a step with no candidate left gives pick -1."""
    lib = _load(mutant)
    C = _c(C, np.float32)
    seeds = _c(seeds, np.int32)
    n, d = C.shape
    nseq = seeds.shape[0]
    assert ((seeds >= 0) & (seeds < n)).all()
    picks = np.empty((nseq, T), np.int32)
    vals = np.empty((nseq, T), np.float64)
    scratch = np.empty((n + 31) // 32, np.uint32)
    lib.orc_div_run(_p(C), n, d, nseq, T, _p(seeds), _p(picks), _p(vals), _p(scratch))
    return picks, vals


def gram_cos(C, threads: int = 1, mutant: int = 0):
    """Full cosine Gram matrix (double) of the rows of C."""
    lib = _load(mutant)
    C = _c(C, np.float32)
    n, d = C.shape
    G = np.empty((n, n), np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        lib.orc_gram_cos(_p(C), n, d, lo, hi, _p(G[lo:hi]))

    shards = _shards(n, threads * 4)
    if threads <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, shards))
    return G


def div_replay(G, seeds, picks, threads: int = 1, mutant: int = 0):
    """Replay recorded picks [nseq, T] against the Gram matrix.  Returns a dict
    of [nseq, T] arrays: bidx, best (cosine of the exact step), gap,
    pick_value (cosine of the recorded pick), pick_ok."""
    lib = _load(mutant)
    G = _c(G, np.float64)
    seeds = _c(seeds, np.int32)
    picks = _c(picks, np.int32)
    n = G.shape[0]
    nseq, T = picks.shape
    out = {k: np.empty((nseq, T), dt) for k, dt in
           (("bidx", np.int32), ("best", np.float64), ("gap", np.float64),
            ("pick_value", np.float64), ("pick_ok", np.int32))}

    def run(lo_hi):
        lo, hi = lo_hi
        scratch = np.empty((n + 31) // 32, np.uint32)
        lib.orc_div_replay(_p(G), n, hi - lo, T, _p(seeds[lo:hi]), _p(picks[lo:hi]),
                           _p(out["bidx"][lo:hi]), _p(out["best"][lo:hi]),
                           _p(out["gap"][lo:hi]), _p(out["pick_value"][lo:hi]),
                           _p(out["pick_ok"][lo:hi]), _p(scratch))

    shards = _shards(nseq, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return out


def div_run_centroid(C, seeds, T: int, threads: int = 1, mutant: int = 0):
    """Diversity sequences with the centroid of the sequence so far as the
    reference.  Returns (picks, cosines to the centroid), both [nseq, T]."""
    lib = _load(mutant)
    C = _c(C, np.float32)
    seeds = _c(seeds, np.int32)
    n, d = C.shape
    nseq = seeds.shape[0]
    picks = np.empty((nseq, T), np.int32)
    vals = np.empty((nseq, T), np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        scratch = np.empty((n + 31) // 32, np.uint32)
        cent = np.empty(d, np.float64)
        lib.orc_div_run_centroid(_p(C), n, d, hi - lo, T, _p(seeds[lo:hi]), _p(picks[lo:hi]),
                                 _p(vals[lo:hi]), _p(scratch), _p(cent))

    shards = _shards(nseq, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return picks, vals


def div_replay_centroid(C, seeds, picks, threads: int = 1, mutant: int = 0):
    """Replay recorded centroid-reference picks [nseq, T] from the table C;
    returns the same dict as :func:`div_replay`."""
    lib = _load(mutant)
    C = _c(C, np.float32)
    seeds = _c(seeds, np.int32)
    picks = _c(picks, np.int32)
    n, d = C.shape
    nseq, T = picks.shape
    out = {k: np.empty((nseq, T), dt) for k, dt in
           (("bidx", np.int32), ("best", np.float64), ("gap", np.float64),
            ("pick_value", np.float64), ("pick_ok", np.int32))}

    def run(lo_hi):
        lo, hi = lo_hi
        scratch = np.empty((n + 31) // 32, np.uint32)
        cent = np.empty(d, np.float64)
        lib.orc_div_replay_centroid(_p(C), n, d, hi - lo, T, _p(seeds[lo:hi]),
                                    _p(picks[lo:hi]), _p(out["bidx"][lo:hi]),
                                    _p(out["best"][lo:hi]), _p(out["gap"][lo:hi]),
                                    _p(out["pick_value"][lo:hi]), _p(out["pick_ok"][lo:hi]),
                                    _p(scratch), _p(cent))

    shards = _shards(nseq, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return out


def dense_as_csr(X):
    """A dense matrix as the CSR matrix holding every entry (row-major)."""
    X = _c(X, np.float32)
    n, d = X.shape
    indptr = np.arange(n + 1, dtype=np.int64) * d
    indices = np.tile(np.arange(d, dtype=np.int32), n)
    return indptr, indices, X.reshape(-1)


def som_update(indptr, indices, values, d: int, bmu, C_old, rows: int, cols: int,
               sigma: float, radius: int, neurons=None, threads: int = 1, mutant: int = 0,
               old_rows=None):
    """Batch SOM update of the requested neurons (all by default).

    Inputs are CSR rows (see :func:`dense_as_csr` for a dense matrix);
    ``C_old`` is the neuron-major codebook (rows*cols x d) before the update,
    or None when ``old_rows`` holds just the requested neurons' old weights.
    Returns (w float64[m, d], mass float64[m, d], den float64[m]) for the
    neurons in ``neurons`` order.
    """
    lib = _load(mutant)
    indptr = _c(indptr, np.int64)
    indices = _c(indices, np.int32)
    values = _c(values, np.float32)
    bmu = _c(bmu, np.int32)
    nc = rows * cols
    assert bmu.shape[0] == indptr.shape[0] - 1
    neurons = np.arange(nc, dtype=np.int32) if neurons is None else _c(neurons, np.int32)
    m = neurons.shape[0]
    if old_rows is None:
        C_old = np.asarray(C_old, np.float32)
        assert C_old.shape == (nc, d)
        old = np.ascontiguousarray(C_old[neurons])
    else:
        old = _c(old_rows, np.float32)
        assert old.shape == (m, d)
    w = np.empty((m, d), np.float64)
    mass = np.empty((m, d), np.float64)
    den = np.empty(m, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        lib.orc_som_update(_p(indptr), _p(indices), _p(values), bmu.shape[0], d, _p(bmu),
                           rows, cols, float(sigma), radius, _p(neurons[lo:hi]), hi - lo,
                           _p(old[lo:hi]), _p(w[lo:hi]), _p(mass[lo:hi]), _p(den[lo:hi]))

    shards = _shards(m, threads)
    if len(shards) <= 1:
        for s in shards:
            run(s)
    else:
        with ThreadPoolExecutor(len(shards)) as ex:
            list(ex.map(run, shards))
    return w, mass, den


def mean_sqrt(d2, mutant: int = 0) -> float:
    """Quantisation error from each input's exact squared distance to its BMU."""
    d2 = _c(d2, np.float64)
    return float(_load(mutant).orc_mean_sqrt(_p(d2), d2.shape[0]))


def mutant_id(mutant: int = 0) -> int:
    return int(_load(mutant).orc_mutant())
