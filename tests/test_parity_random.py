"""Seeded random cases across the entry points (GPU parity, through the C ABI).

Shapes, feature counts, metrics and value distributions are drawn from a
seeded generator, so each case is fixed and reproducible; every result is
held to the same bar as the hand-picked tests (tests/parity.py): the dense
and sparse searches against the oracle's exact scan, diversity chains
against the oracle's step-by-step replay.  The case counts (24, 12, 8) can
be raised for a longer sweep with VS_RANDOM_DENSE, VS_RANDOM_CSR and
VS_RANDOM_DIVERSITY.
"""
import os

import numpy as np
import pytest

import synth
from test_parity_dense import assert_parity
from test_parity_div_csr import csr_case, csr_parity, gpu_chain, validate_chain

pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _draws(key, count):
    (r,) = synth.rng_children(20000 + key, 1)
    return r, count


@pytest.mark.parametrize("case", range(int(os.environ.get("VS_RANDOM_DENSE", "24"))))
def test_random_dense(case):
    r, _ = _draws(case, 1)
    nq = int(r.integers(1, 300))
    nc = int(r.integers(1, 2000))
    d = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 300)), int(r.integers(300, 800))]))
    metric = int(r.integers(0, 4))
    dist = "unit" if metric in (2, 3) else str(r.choice(["normal", "uniform", "int"]))
    Q, C = synth.dense_case(nq, nc, d, dist, key=30000 + case)
    assert_parity(Q, C, metric)


@pytest.mark.parametrize("case", range(int(os.environ.get("VS_RANDOM_CSR", "12"))))
def test_random_csr(case):
    r, _ = _draws(100 + case, 1)
    nq = int(r.integers(1, 120))
    d = int(r.integers(8, 3000))
    nc = int(r.integers(1, 1500))
    p = float(r.uniform(0.005, 0.1))
    metric = int(r.integers(0, 4))
    indptr, indices, values, CT = csr_case(nq, d, nc, p, key=31000 + case)
    if metric in (2, 3):
        # a cosine needs a non-zero query: keep the non-empty rows
        counts = np.diff(indptr)
        if not (counts > 0).any():
            counts[0] = 0
            indptr = np.array([0, 1], np.int32)
            indices, values = np.array([0], np.int32), np.array([1.0], np.float32)
        else:
            indptr = np.concatenate([[0], np.cumsum(counts[counts > 0])]).astype(np.int32)
    csr_parity(indptr, indices, values, CT, metric)


@pytest.mark.parametrize("case", range(int(os.environ.get("VS_RANDOM_DIVERSITY", "8"))))
def test_random_diversity_chain(case):
    r, _ = _draws(200 + case, 1)
    n = int(r.integers(20, 1500))
    d = int(r.choice([int(r.integers(2, 64)), int(r.integers(64, 769))]))
    nseq = int(r.integers(1, 300))
    steps = int(r.integers(1, min(n, 40)))
    C = synth.dense_case(1, n, d, "unit", key=32000 + case)[1]
    seeds = r.choice(n, nseq, replace=nseq > n).astype(np.int32)
    picks, scores, masks = gpu_chain(C, seeds, steps)
    fails, _ = validate_chain(C, seeds, picks, scores, masks)
    assert not fails, fails
