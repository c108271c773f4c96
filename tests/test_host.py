"""Host-side checks of the C ABI (no GPU needed, no compute call).

* libvs.so loads and exports every function include/vs.h declares;
* argument validation returns the documented status before anything is
  enqueued (fake, never-dereferenced addresses are enough for that);
* the cache-sized tile rule reproduces the figures printed in "Issue 9-014:
  Tile Diversity Shader Inner Loop For L2 Cache Locality" ("Intended
  Behavior", "FP16 storage path").
"""
import ctypes
import os
import re
import subprocess

import pytest

import farthest_vector_search_amd as vs
from goldens import tile_rule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vs.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vs.LIB_PATH):
        from farthest_vector_search_amd.build import build
        build(verbose=False)
    return vs.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    fns = header_functions()
    for name in ("vs_bmu_search", "vs_bmu_search_csr", "vs_bmu_search_csr_blocked",
                 "vs_csr_block_codebook", "vs_diversity_step", "vs_candidate_norms",
                 "vs_tile_rows", "vs_status_str"):
        assert name in fns
    assert sorted(vs.EXPORTS) == fns


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", vs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    # nothing but the C ABI is exported from the library's own code
    assert not [s for s in exported if s.startswith("_ZN2vs")]


def test_status_strings(L):
    for code in range(9):
        s = L.vs_status_str(code).decode()
        assert s and s != "unknown status"
    assert L.vs_status_str(99).decode() == "unknown status"
    assert b"gfx950" in L.vs_version()


FAKE = 0x10000  # 256-byte aligned, never dereferenced by argument checks


def _P(x):
    return ctypes.c_void_p(x)


def dense_call(L, Q=FAKE, C=FAKE, nq=4, nc=8, d=4, metric=0, idx=FAKE, score=FAKE,
               ws=FAKE, ws_bytes=1 << 20):
    return L.vs_bmu_search(_P(Q), _P(C), nq, nc, d, metric, _P(idx), _P(score), _P(ws),
                           ws_bytes, None)


def test_dense_validation(L):
    assert dense_call(L, metric=4) == 3
    assert dense_call(L, metric=-1) == 3
    assert dense_call(L, nq=-1) == 2
    assert dense_call(L, nc=0) == 2
    assert dense_call(L, nc=2 ** 31) == 2
    assert dense_call(L, d=0) == 2
    assert dense_call(L, nq=0, Q=0, C=0, idx=0, ws=0) == 0  # empty query set: no-op
    assert dense_call(L, Q=0) == 1
    assert dense_call(L, C=0) == 1
    assert dense_call(L, idx=0) == 1
    assert dense_call(L, ws=0) == 1
    assert dense_call(L, Q=FAKE + 2) == 5
    assert dense_call(L, score=FAKE + 1) == 5
    assert dense_call(L, ws=FAKE + 8) == 5
    need = L.vs_bmu_search_workspace(4, 8, 4, 0)
    assert need >= 4 * 8
    assert dense_call(L, ws_bytes=need - 1) == 4


def test_unfused_validation(L):
    def call(Q=FAKE, C=FAKE, nq=4, nc=8, d=4, metric=0, idx=FAKE, score=FAKE, S=FAKE, ld=8,
             ws=FAKE, ws_bytes=1 << 20):
        return L.vs_bmu_search_unfused(_P(Q), _P(C), nq, nc, d, metric, _P(idx), _P(score),
                                       _P(S), ld, _P(ws), ws_bytes, None)
    assert call(metric=4) == 3
    assert call(ld=7) == 2
    assert call(ld=10) == 2  # not a multiple of 4
    assert call(nq=0, Q=0) == 0
    assert call(S=0) == 1
    assert call(S=FAKE + 4) == 5
    assert call(d=1000) == 7
    assert call(ws_bytes=8) == 4


def test_workspace_sizes(L):
    # keys (8 B per query) always; squared L2 adds query and candidate norms
    # keys[nq] u64 | qn[nq] f32 | cn[nc] f32, each 256-byte aligned
    assert L.vs_bmu_search_workspace(1000, 2100, 64, 2) == 8192
    assert L.vs_bmu_search_workspace(1000, 2100, 64, 0) == 8192 + 4096 + 8448
    # a search the small path may take: nq * ceil(nc / 32) keys + nq norms
    assert L.vs_bmu_search_workspace(1000, 500, 64, 2) == 1000 * 16 * 8 + 4096
    assert L.vs_bmu_search_workspace(1000, 500, 64, 0) == 1000 * 16 * 8 + 4096
    assert L.vs_bmu_search_workspace(1000, 500, 300, 0) == 8192 + 4096 + 2048  # d > 256
    assert L.vs_diversity_step_workspace(8359, 768, 3584) == 28672
    assert L.vs_bmu_search_workspace(-1, 5, 4, 0) == 0


def test_csr_validation(L):
    def call(indptr=FAKE, indices=FAKE, values=FAKE, nq=3, nnz=10, CT=FAKE, nc=16, ld=None,
             d=8, metric=0, idx=FAKE, score=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_bmu_search_csr(_P(indptr), _P(indices), _P(values), nq, nnz, _P(CT), nc,
                                   nc if ld is None else ld, d, metric, _P(idx), _P(score),
                                   _P(ws), ws_bytes, None)
    assert call(metric=7) == 3
    assert call(nnz=-1) == 2
    assert call(nc=0) == 2
    assert call(ld=15) == 2  # row stride below nc
    assert call(nq=0, indptr=0) == 0
    assert call(indptr=0) == 1
    assert call(indices=0) == 1
    assert call(nnz=0, indices=0, values=0, ws_bytes=0) == 4  # empty arrays allowed
    assert call(CT=FAKE + 1) == 5
    assert call(ws_bytes=10) == 4


def test_csr_blocked_validation(L):
    assert L.vs_csr_blocked_bytes(1, 1) == 256
    assert L.vs_csr_blocked_bytes(65, 10) == 2 * 64 * 10 * 4
    assert L.vs_csr_blocked_bytes(0, 10) == 0
    assert L.vs_csr_blocked_bytes(10, 0) == 0
    blk = lambda CT=FAKE, nc=16, ld=16, d=8, CB=FAKE: L.vs_csr_block_codebook(
        _P(CT), nc, ld, d, _P(CB), None)
    assert blk(ld=15) == 2
    assert blk(nc=0) == 2
    assert blk(d=0) == 2
    assert blk(CT=0) == 1
    assert blk(CB=0) == 1
    assert blk(CB=FAKE + 2) == 5

    def call(indptr=FAKE, indices=FAKE, values=FAKE, nq=3, nnz=10, CB=FAKE, nc=16, d=8,
             metric=0, idx=FAKE, score=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_bmu_search_csr_blocked(_P(indptr), _P(indices), _P(values), nq, nnz, _P(CB),
                                           nc, d, metric, _P(idx), _P(score), _P(ws), ws_bytes,
                                           None)
    assert call(metric=5) == 3
    assert call(nc=0) == 2
    assert call(d=0) == 2
    assert call(nq=0, indptr=0) == 0
    assert call(CB=0) == 1
    assert call(CB=FAKE + 1) == 5
    assert call(ws_bytes=10) == 4


def test_csr_f16_validation(L):
    assert L.vs_csr_blocked_f16_bytes(1, 1) == 256
    assert L.vs_csr_blocked_f16_bytes(129, 10) == 2 * 128 * 10 * 2
    assert L.vs_csr_blocked_f16_bytes(0, 3) == 0
    blk = lambda CT=FAKE, nc=16, ld=16, d=8, CB=FAKE: L.vs_csr_block_codebook_f16(
        _P(CT), nc, ld, d, _P(CB), None)
    assert blk(ld=15) == 2
    assert blk(CT=0) == 1
    assert blk(CB=FAKE + 8) == 5  # 16-byte alignment

    def call(indptr=FAKE, indices=FAKE, values=FAKE, nq=3, nnz=10, CB=FAKE, nc=16, d=8,
             metric=0, idx=FAKE, score=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_bmu_search_csr_blocked_f16(_P(indptr), _P(indices), _P(values), nq, nnz,
                                               _P(CB), nc, d, metric, _P(idx), _P(score),
                                               _P(ws), ws_bytes, None)
    assert call(metric=9) == 3
    assert call(nc=0) == 2
    assert call(CB=0) == 1
    assert call(CB=FAKE + 8) == 5
    assert call(ws_bytes=10) == 4


def test_diversity_gram_validation(L):
    gram = lambda C=FAKE, n=100, d=8, G=FAKE, ld=100: L.vs_diversity_gram(_P(C), n, d, _P(G),
                                                                           ld, None)
    assert gram(ld=99) == 2
    assert gram(ld=102) == 2  # not a multiple of 4
    assert gram(n=0) == 2
    assert gram(C=0) == 1
    assert gram(G=FAKE + 4) == 5
    assert gram(d=770) == 7  # beyond the register-resident kernel
    assert gram(d=6) == 7

    def step(G=FAKE, n=100, ld=100, pick=FAKE, mask=FAKE, nseq=5, idx=FAKE, score=FAKE):
        return L.vs_diversity_step_gram(_P(G), n, ld, _P(pick), _P(mask), nseq, _P(idx),
                                        _P(score), None)
    assert step(ld=98) == 2
    assert step(nseq=0, G=0) == 0
    assert step(mask=0) == 1
    assert step(G=FAKE + 8) == 5
    assert step(pick=FAKE + 2) == 5


def test_diversity_validation(L):
    def call(C=FAKE, n=100, d=8, pick=FAKE, mask=FAKE, nseq=5, idx=FAKE, score=FAKE, ws=FAKE,
             ws_bytes=1 << 20):
        return L.vs_diversity_step(_P(C), n, d, _P(pick), _P(mask), nseq, _P(idx), _P(score),
                                   _P(ws), ws_bytes, None)
    assert call(n=0) == 2
    assert call(d=-3) == 2
    assert call(nseq=0, C=0) == 0
    assert call(mask=0) == 1
    assert call(pick=0) == 1
    assert call(mask=FAKE + 2) == 5
    assert call(ws_bytes=8) == 4


def test_diversity_reference_validation(L):
    def step(C=FAKE, n=100, d=8, Q=FAKE, mask=FAKE, nseq=5, idx=FAKE, score=FAKE, ws=FAKE,
             ws_bytes=1 << 20):
        return L.vs_diversity_step_ref(_P(C), n, d, _P(Q), _P(mask), nseq, _P(idx), _P(score),
                                       _P(ws), ws_bytes, None)
    assert step(n=0) == 2
    assert step(d=0) == 2
    assert step(nseq=-1) == 2
    assert step(nseq=0, Q=0) == 0
    assert step(Q=0) == 1
    assert step(mask=0) == 1
    assert step(Q=FAKE + 2) == 5
    assert step(ws=FAKE + 8) == 5
    assert step(ws_bytes=8) == 4

    def acc(C=FAKE, n=100, d=8, pick=FAKE, Q=FAKE, nseq=5):
        return L.vs_diversity_accumulate(_P(C), n, d, _P(pick), _P(Q), nseq, None)
    assert acc(n=0) == 2
    assert acc(d=0) == 2
    assert acc(nseq=0, C=0) == 0
    assert acc(pick=0) == 1
    assert acc(Q=0) == 1
    assert acc(pick=FAKE + 1) == 5


def test_diversity_run_validation(L):
    def run(C=FAKE, n=100, d=8, seeds=FAKE, mask=FAKE, nseq=5, steps=3, picks=FAKE, scores=FAKE,
            ws=FAKE, ws_bytes=1 << 20):
        return L.vs_diversity_run(_P(C), n, d, _P(seeds), _P(mask), nseq, steps, _P(picks),
                                  _P(scores), _P(ws), ws_bytes, None)
    assert run(steps=-1) == 2
    assert run(n=0) == 2
    assert run(steps=0, seeds=0) == 0
    assert run(seeds=0) == 1
    assert run(picks=0) == 1
    assert run(ws_bytes=8) == 4
    # every check of the steps is made before the first step is enqueued
    assert run(C=0) == 1
    assert run(mask=0) == 1
    assert run(ws=0) == 1
    assert run(mask=FAKE + 2) == 5
    assert run(scores=FAKE + 1) == 5
    assert run(ws=FAKE + 8) == 5
    assert run(d=0) == 2

    def run_gram(G=FAKE, n=100, ldg=128, seeds=FAKE, R=0, ldr=0, mask=FAKE, nseq=5, steps=3,
                 picks=FAKE, scores=FAKE):
        return L.vs_diversity_run_gram(_P(G), n, ldg, _P(seeds), _P(R), ldr, _P(mask), nseq,
                                       steps, _P(picks), _P(scores), None)
    assert run_gram(steps=-2) == 2
    assert run_gram(ldg=99) == 2
    assert run_gram(R=FAKE, ldr=98) == 2
    assert run_gram(R=FAKE, ldr=102) == 2
    assert run_gram(nseq=0, seeds=0) == 0
    assert run_gram(picks=0) == 1
    assert run_gram(R=FAKE + 4, ldr=128) == 5
    # every check of the steps is made before anything (clearing R) is enqueued
    assert run_gram(ldg=130) == 2
    assert run_gram(G=0, R=FAKE, ldr=128) == 1
    assert run_gram(mask=0, R=FAKE, ldr=128) == 1
    assert run_gram(G=FAKE + 4, R=FAKE, ldr=128) == 5
    assert run_gram(mask=FAKE + 2, R=FAKE, ldr=128) == 5


def test_diversity_run_ref_validation(L):
    def run(C=FAKE, n=100, d=8, seeds=FAKE, Q=FAKE, mask=FAKE, nseq=5, steps=3, picks=FAKE,
            scores=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_diversity_run_ref(_P(C), n, d, _P(seeds), _P(Q), _P(mask), nseq, steps,
                                      _P(picks), _P(scores), _P(ws), ws_bytes, None)
    assert run(steps=-1) == 2
    assert run(d=0) == 2
    assert run(steps=0, Q=0) == 0
    assert run(Q=0) == 1
    assert run(seeds=0) == 1
    assert run(Q=FAKE + 2) == 5
    # every check of the steps is made before Q is cleared and seeded
    assert run(mask=0) == 1
    assert run(ws=0) == 1
    assert run(ws=FAKE + 16) == 5
    assert run(picks=FAKE + 2) == 5
    assert run(ws_bytes=8) == 4


def test_fp16_epoch_validation(L):
    F = ctypes.c_float
    assert L.vs_csr_blocked_to_f16(_P(FAKE), 0, 8, _P(FAKE), None) == 2
    assert L.vs_csr_blocked_to_f16(_P(FAKE), 10, 0, _P(FAKE), None) == 2
    assert L.vs_csr_blocked_to_f16(None, 10, 8, _P(FAKE), None) == 1
    assert L.vs_csr_blocked_to_f16(_P(FAKE), 10, 8, _P(FAKE + 8), None) == 5

    def ep(indptr=FAKE, indices=FAKE, values=FAKE, n=10, nnz=30, CB=FAKE, CB16=FAKE, rows=4,
           cols=4, d=8, sigma=1.0, R=2, bmu=FAKE, score=FAKE, qe=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_som_epoch_csr_f16(_P(indptr), _P(indices), _P(values), n, nnz, _P(CB),
                                      _P(CB16), rows, cols, d, F(sigma), R, _P(bmu), _P(score),
                                      _P(qe), _P(ws), ws_bytes, None)
    assert ep(R=-1) == 2
    assert ep(CB16=0) == 1
    assert ep(CB=0) == 1
    assert ep(qe=FAKE + 4) == 5
    assert ep(ws_bytes=10) == 4


def test_som_validation(L):
    F = ctypes.c_float
    assert L.vs_som_update_workspace(0, 4, 8) == 0
    assert L.vs_som_update_workspace(4, 0, 8) == 0
    assert L.vs_som_update_workspace(4, 4, 0) == 0
    # two 64-neuron-rounded float buffers, three count/denominator arrays, the 1-D weights
    assert L.vs_som_update_workspace(4, 4, 8) == 2 * 64 * 8 * 4 + 3 * 256 + 256
    assert L.vs_som_epoch_workspace(-1, 4, 4, 8) == 0
    assert L.vs_som_epoch_workspace(10, 4, 4, 8) > L.vs_som_update_workspace(4, 4, 8)
    assert L.vs_som_epoch_csr_workspace(10, 4, 4, 8) > L.vs_som_update_workspace(4, 4, 8)

    def upd(X=FAKE, n=10, d=8, bmu=FAKE, C=FAKE, rows=4, cols=4, sigma=1.0, R=2, ws=FAKE,
            ws_bytes=1 << 20):
        return L.vs_som_update(_P(X), n, d, _P(bmu), _P(C), rows, cols, F(sigma), R, _P(ws),
                               ws_bytes, None)
    assert upd(sigma=0.0) == 2
    assert upd(sigma=-1.0) == 2
    assert upd(sigma=float("nan")) == 2
    assert upd(sigma=float("inf")) == 2
    assert upd(R=-1) == 2
    assert upd(sigma=0.25, R=3) == 2      # window beyond 8 sigma
    assert upd(sigma=0.01, R=0, ws_bytes=100) == 4  # R = 0 is the per-neuron mean at any sigma
    assert upd(rows=0) == 2
    assert upd(n=-1) == 2
    assert upd(n=0, X=0) == 0             # nothing to do
    assert upd(X=0) == 1
    assert upd(bmu=0) == 1
    assert upd(C=FAKE + 2) == 5
    assert upd(ws=FAKE + 16) == 5
    assert upd(ws_bytes=100) == 4

    def upd_csr(indptr=FAKE, indices=FAKE, values=FAKE, n=10, nnz=30, bmu=FAKE, CB=FAKE,
                rows=4, cols=4, d=8, sigma=1.0, R=2, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_som_update_csr(_P(indptr), _P(indices), _P(values), n, nnz, _P(bmu), _P(CB),
                                   rows, cols, d, F(sigma), R, _P(ws), ws_bytes, None)
    assert upd_csr(d=0) == 2
    assert upd_csr(nnz=-1) == 2
    assert upd_csr(indices=0) == 1
    assert upd_csr(nnz=0, indices=0, values=0, ws_bytes=10) == 4
    assert upd_csr(values=FAKE + 1) == 5
    assert upd_csr(ws_bytes=10) == 4

    assert L.vs_som_qe(_P(FAKE), -1, _P(FAKE), None) == 2
    assert L.vs_som_qe(_P(FAKE), 5, None, None) == 1
    assert L.vs_som_qe(None, 5, _P(FAKE), None) == 1
    assert L.vs_som_qe(_P(FAKE), 5, _P(FAKE + 4), None) == 5

    def ep(X=FAKE, n=10, d=8, C=FAKE, rows=4, cols=4, sigma=1.0, R=2, bmu=FAKE, score=FAKE,
           qe=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_som_epoch(_P(X), n, d, _P(C), rows, cols, F(sigma), R, _P(bmu), _P(score),
                              _P(qe), _P(ws), ws_bytes, None)
    assert ep(sigma=0.0) == 2
    assert ep(cols=0) == 2
    assert ep(bmu=0) == 1
    assert ep(score=0) == 1
    assert ep(qe=FAKE + 4) == 5
    assert ep(ws_bytes=10) == 4

    def ep_csr(indptr=FAKE, indices=FAKE, values=FAKE, n=10, nnz=30, CB=FAKE, rows=4, cols=4,
               d=8, sigma=1.0, R=2, bmu=FAKE, score=FAKE, qe=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return L.vs_som_epoch_csr(_P(indptr), _P(indices), _P(values), n, nnz, _P(CB), rows, cols,
                                  d, F(sigma), R, _P(bmu), _P(score), _P(qe), _P(ws), ws_bytes,
                                  None)
    assert ep_csr(R=-2) == 2
    assert ep_csr(CB=0) == 1
    assert ep_csr(ws_bytes=10) == 4


def test_norms_validation(L):
    assert L.vs_candidate_norms(_P(FAKE), 10, 0, 0, _P(FAKE), None) == 2
    assert L.vs_candidate_norms(_P(0), 10, 4, 0, _P(FAKE), None) == 1
    assert L.vs_candidate_norms(_P(FAKE + 1), 10, 4, 0, _P(FAKE), None) == 5
    assert L.vs_candidate_norms(_P(0), 0, 4, 0, _P(0), None) == 0


@pytest.mark.parametrize("case", tile_rule(), ids=lambda c: f"{c[1]}x{c[2]}B")
def test_tile_rule_matches_page_figures(L, case):
    cache, d, b, approx = case
    rows = L.vs_tile_rows(cache, d, b)
    assert abs(rows - approx) <= 0.10 * approx
    # the rule itself: the largest tile that fits 85 % of the cache
    assert rows * d * b <= 0.85 * cache < (rows + 1) * d * b


def test_tile_rule_edges(L):
    assert L.vs_tile_rows(0, 768, 4) == 0
    assert L.vs_tile_rows(100, 0, 4) == 0
    assert L.vs_tile_rows(100, 768, 4) == 1  # at least one row
    # MI355X L2 per XCD (4 MiB) at the workload dimensions
    assert L.vs_tile_rows(4 << 20, 256, 4) == 3481
    assert L.vs_tile_rows(4 << 20, 768, 4) == 1160
