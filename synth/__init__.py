"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module is shared by the tests, the benchmark and the smoke check.  It
holds random-number generation and data layout only: no distance, no
arg-reduction, nothing of the method's arithmetic.  Both the HIP path and the
oracle receive the arrays produced here.

Sources of the shapes (cited by page title and section):
  * "From 80x to 385x: A Best-Matching-Unit Search at the L2 Roof ..."
    (summary), abstract and section 4.1: SOM maps from 32x32 to 512x512
    neurons, sparse article vectors, feature-major codebook (section 3).
  * "Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality",
    "Current Behavior": a table of 8,359 embeddings of 768 dimensions and
    3,584 workgroups (one per sequence).

Recipe (readings where the configurations leave a choice open):
  * seeds: numpy ``default_rng(SeedSequence(20261202 + k))`` for workload k,
    spawned into independent children per array;
  * "uniform[0,1)": ``rng.random(dtype=float32)`` (stays below 1 in fp32);
  * "N(mu, s)": ``s * rng.standard_normal(dtype=float32)`` (s is the std);
  * "rows L2-normalised": norms taken in float64, division in float64, then
    rounded to float32;
  * sparse rows: every column kept independently with probability 0.01,
    columns ascending and unique, values lognormal(0, 1), row normalised;
    an empty row stays empty;
  * the sparse-workload codebook (left unspecified) is uniform[0,1) with
    every neuron (column of the feature-major matrix) normalised;
  * diversity seeds: ``rng.choice(n, nseq, replace=False)``.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202


def rng_children(key: int, n: int):
    """n independent generators for workload ``key``."""
    ss = np.random.SeedSequence(BASE_SEED + int(key))
    return [np.random.default_rng(c) for c in ss.spawn(n)]


def uniform01(rng, shape):
    return rng.random(shape, dtype=np.float32)


def normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normalize_rows(x: np.ndarray, block: int = 1 << 16) -> np.ndarray:
    """Rows scaled to unit L2 norm in float64, stored as float32 (in place on
    a float32 copy, processed in row blocks to bound memory)."""
    out = np.empty(x.shape, np.float32)
    for lo in range(0, x.shape[0], block):
        b = x[lo:lo + block].astype(np.float64)
        nrm = np.sqrt((b * b).sum(axis=1, keepdims=True))
        nrm[nrm == 0] = 1.0
        out[lo:lo + block] = (b / nrm).astype(np.float32)
    return out


def normalize_columns(x: np.ndarray, block: int = 512) -> None:
    """Columns of a float32 matrix scaled to unit L2 norm in float64, in place."""
    rows = x.shape[0]
    acc = np.zeros(x.shape[1], np.float64)
    for lo in range(0, rows, block):
        b = x[lo:lo + block].astype(np.float64)
        acc += (b * b).sum(axis=0)
    nrm = np.sqrt(acc)
    nrm[nrm == 0] = 1.0
    for lo in range(0, rows, block):
        b = x[lo:lo + block].astype(np.float64)
        x[lo:lo + block] = (b / nrm).astype(np.float32)


def sparse_rows(rng, nrows: int, ncols: int, p: float = 0.01, block: int = 1024):
    """CSR (indptr int32, indices int32, values float32) with Bernoulli(p)
    column pattern, lognormal(0,1) values, each non-empty row unit-norm."""
    ptr = [np.zeros(1, np.int64)]
    idx_parts, val_parts = [], []
    total = 0
    for lo in range(0, nrows, block):
        hi = min(nrows, lo + block)
        keep = rng.random((hi - lo, ncols), dtype=np.float32) < np.float32(p)
        r, c = np.nonzero(keep)  # row-major order: columns ascending per row
        counts = np.bincount(r, minlength=hi - lo)
        v = rng.lognormal(0.0, 1.0, size=c.shape[0])
        # per-row norm in float64
        sq = np.bincount(r, weights=v * v, minlength=hi - lo)
        nrm = np.sqrt(sq)
        nrm[nrm == 0] = 1.0
        v = (v / nrm[r]).astype(np.float32)
        idx_parts.append(c.astype(np.int32))
        val_parts.append(v)
        ptr.append(total + np.cumsum(counts))
        total += int(counts.sum())
    indptr = np.concatenate(ptr).astype(np.int32)
    indices = np.concatenate(idx_parts) if idx_parts else np.zeros(0, np.int32)
    values = np.concatenate(val_parts) if val_parts else np.zeros(0, np.float32)
    return indptr, indices, values


# ------------------------------------------------------------ workloads --

WORKLOADS = {
    1: dict(name="bmu_dense_32x32_map", kind="dense", nq=256, nc=1024, d=64, metric=0),
    2: dict(name="bmu_dense_128x128_map", kind="dense", nq=65536, nc=16384, d=256, metric=0),
    3: dict(name="diversity_8359x768", kind="diversity", n=8359, d=768, nseq=3584, steps=64),
    4: dict(name="bmu_csr_256x256_map", kind="csr", nq=32768, d=16384, nc=65536, metric=0),
    5: dict(name="bmu_dense_512x512_map", kind="dense", nq=65536, nc=262144, d=256, metric=0,
            oracle_subset=1024),
}


def workload(k: int) -> dict:
    """Inputs of workload k (numpy arrays) plus its description."""
    w = dict(WORKLOADS[k])
    if k == 1:
        rq, rc = rng_children(k, 2)
        w["Q"] = uniform01(rq, (w["nq"], w["d"]))
        w["C"] = uniform01(rc, (w["nc"], w["d"]))
    elif k == 2:
        rq, rc = rng_children(k, 2)
        w["Q"] = normal(rq, (w["nq"], w["d"]), 1.0)
        w["C"] = normal(rc, (w["nc"], w["d"]), 0.5)
    elif k == 3:
        rc, rs = rng_children(k, 2)
        w["C"] = normalize_rows(normal(rc, (w["n"], w["d"])))
        w["seeds"] = rs.choice(w["n"], w["nseq"], replace=False).astype(np.int32)
    elif k == 4:
        rq, rc = rng_children(k, 2)
        w["indptr"], w["indices"], w["values"] = sparse_rows(rq, w["nq"], w["d"], 0.01)
        CT = uniform01(rc, (w["d"], w["nc"]))
        normalize_columns(CT)
        w["CT"] = CT
    elif k == 5:
        rq, rc, rs = rng_children(k, 3)
        w["Q"] = normal(rq, (w["nq"], w["d"]))
        w["C"] = normal(rc, (w["nc"], w["d"]))
        w["subset"] = np.sort(rs.choice(w["nq"], w["oracle_subset"], replace=False)).astype(np.int64)
    return w


def sample_queries(nq: int, count: int, key: int) -> np.ndarray:
    """Seeded, sorted sample of query indices (for spot checks at full size)."""
    (r,) = rng_children(1000 + key, 1)
    count = min(count, nq)
    return np.sort(r.choice(nq, count, replace=False)).astype(np.int64)


def dense_case(nq: int, nc: int, d: int, dist: str = "normal", key: int = 0):
    """Small dense case: Q [nq, d], C [nc, d] float32 ('normal', 'uniform',
    'unit' = normal rows normalised, 'int' = small integers)."""
    rq, rc = rng_children(5000 + key, 2)
    if dist == "uniform":
        return uniform01(rq, (nq, d)), uniform01(rc, (nc, d))
    if dist == "unit":
        return normalize_rows(normal(rq, (nq, d))), normalize_rows(normal(rc, (nc, d)))
    if dist == "int":
        return (rq.integers(-8, 9, (nq, d)).astype(np.float32),
                rc.integers(-8, 9, (nc, d)).astype(np.float32))
    return normal(rq, (nq, d)), normal(rc, (nc, d))


def random_indices(n: int, hi: int, key: int = 0) -> np.ndarray:
    """int32[n] uniform in [0, hi) (e.g. a BMU assignment handed to an update)."""
    (r,) = rng_children(8000 + key, 1)
    return r.integers(0, hi, n).astype(np.int32)


def random_mask(nq: int, nc: int, frac: float, key: int = 0) -> np.ndarray:
    """uint32 mask words [nq, ceil(nc/32)], each candidate excluded with
    probability ``frac``; bits at or above nc are left clear."""
    (r,) = rng_children(7000 + key, 1)
    bits = r.random((nq, nc)) < frac
    W = (nc + 31) // 32
    padded = np.zeros((nq, W * 32), bool)
    padded[:, :nc] = bits
    w = padded.reshape(nq, W, 32).astype(np.uint64)
    shifts = np.arange(32, dtype=np.uint64)
    return (w << shifts).sum(axis=2).astype(np.uint32)
