"""GPU parity of the diversity step and the sparse-query search.

Diversity: the GPU runs the whole chain of steps on the device (each step's
picks feed the next as reference rows); the oracle then replays the GPU's
prefix step by step against the fp64 cosine Gram matrix and validates every
pick with the rule of tests/parity.py.  The masks must end up holding
exactly the seed plus the picks.

Sparse: CSR queries over a feature-major codebook, checked against the
oracle's sparse scan (itself pinned to the dense scan on densified rows).
"""
import numpy as np
import pytest

import oracle
import synth
from goldens import csr_cases, diversity_walk
from parity import check

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import farthest_vector_search_amd as vs  # noqa: E402


def dev():
    return torch.device("cuda:0")


def T(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def seed_masks(n, seeds):
    W = (n + 31) // 32
    m = np.zeros((len(seeds), W), np.uint32)
    for s, j in enumerate(seeds):
        m[s, j // 32] |= np.uint32(1 << (j % 32))
    return m


def gpu_chain(C, seeds, steps):
    """Run `steps` diversity steps on the GPU; returns picks, scores, masks."""
    Cd = T(C)
    nseq = len(seeds)
    mask = T(seed_masks(C.shape[0], seeds).view(np.int32))
    last = T(np.asarray(seeds, np.int32))
    picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    scores = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    ws = torch.empty(vs.lib().vs_diversity_step_workspace(C.shape[0], C.shape[1], nseq),
                     dtype=torch.uint8, device=dev())
    for t in range(steps):
        vs.vs_diversity_step(Cd, last, mask, idx_out=picks[t], score_out=scores[t], workspace=ws)
        last = picks[t]
    torch.cuda.synchronize()
    return (picks.cpu().numpy().T.copy(), scores.cpu().numpy().T.copy(),
            mask.cpu().numpy().view(np.uint32))


def validate_chain(C, seeds, picks, scores, masks, threads=8):
    G = oracle.gram_cos(C, threads=threads)
    rep = oracle.div_replay(G, seeds, picks, threads=threads)
    fails = []
    live = rep["bidx"] >= 0
    # every pick legal where something was left; -1 exactly where nothing was
    if not (rep["pick_ok"][live] == 1).all():
        fails.append("illegal pick (masked or out of range)")
    if not (picks[~live] == -1).all():
        fails.append("pick where nothing was left")
    nseq, steps = picks.shape
    floor = 1e-2
    f, stats = check(picks.reshape(-1), scores.reshape(-1), rep["bidx"].reshape(-1),
                     rep["best"].reshape(-1), rep["gap"].reshape(-1), 3, floor,
                     lambda r, c: rep["pick_value"].reshape(-1)[r],
                     legal=lambda r, c: rep["pick_ok"].reshape(-1)[r] == 1)
    fails += f
    # masks: seed plus every pick, nothing else
    n = C.shape[0]
    exp = seed_masks(n, seeds)
    for s in range(nseq):
        for p in picks[s]:
            if p >= 0:
                exp[s, p // 32] |= np.uint32(1 << (p % 32))
    if not np.array_equal(exp, masks):
        fails.append("final masks differ from seed + picks")
    for s in range(nseq):
        row = picks[s][picks[s] >= 0]
        if len(np.unique(row)) != len(row) or seeds[s] in row:
            fails.append(f"sequence {s} repeats a row")
            break
    return fails, stats


@pytest.fixture(params=["q16", "tiled"])
def div_kernel(request, monkeypatch):
    """Run a diversity test with each kernel that implements the step: 16
    sequences per wave in registers (d <= 768, d % 4 == 0) and the LDS-tiled
    kernel (any d)."""
    monkeypatch.setenv("VS_DIV_KERNEL", request.param)
    return request.param


def gpu_chain_gram(C, seeds, steps):
    """The same chain as gpu_chain, from the cached Gram matrix."""
    Cd = T(C)
    nseq = len(seeds)
    mask = T(seed_masks(C.shape[0], seeds).view(np.int32))
    last = T(np.asarray(seeds, np.int32))
    picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    scores = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    G = vs.vs_diversity_gram(Cd)
    for t in range(steps):
        vs.vs_diversity_step_gram(G, last, mask, idx_out=picks[t], score_out=scores[t])
        last = picks[t]
    torch.cuda.synchronize()
    return (picks.cpu().numpy().T.copy(), scores.cpu().numpy().T.copy(),
            mask.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("n,d,nseq,steps", [(40, 4, 5, 41), (300, 64, 129, 20),
                                            (129, 768, 70, 6), (3000, 128, 300, 4),
                                            (700, 500, 520, 5)])
def test_diversity_gram_matches_step(n, d, nseq, steps, monkeypatch):
    """Steps from the cached Gram matrix equal the per-step MFMA scan bit for
    bit (picks, scores, masks): each Gram entry is the dot product the scan
    ranks, and the masked arg-min rule is the same."""
    monkeypatch.setenv("VS_DIV_KERNEL", "q16")
    C = synth.dense_case(1, n, d, "unit", key=7 * n + d)[1]
    (r,) = synth.rng_children(950 + n, 1)
    seeds = r.choice(n, nseq, replace=nseq > n).astype(np.int32)
    a = gpu_chain(C, seeds, steps)
    b = gpu_chain_gram(C, seeds, steps)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2], b[2])
    fails, _ = validate_chain(C, seeds, *b)
    assert not fails, fails


def test_diversity_gram_entries():
    """The cached Gram matrix against the oracle's fp64 cosine Gram matrix
    (unit rows), within fp32 rounding of a 768-term dot product."""
    C = synth.dense_case(1, 500, 768, "unit", key=99)[1]
    G = vs.vs_diversity_gram(T(C)).cpu().numpy()
    ref = oracle.gram_cos(C, threads=8)
    assert np.abs(G.astype(np.float64) - ref).max() <= 2e-6


@pytest.mark.parametrize("n,d", [(40, 4), (129, 300), (700, 768), (1000, 260), (2049, 16)])
def test_diversity_gram_symmetric_build(n, d):
    """The Gram build computes the tiles at or right of each 128-row block's
    own rows and writes the rest as their transpose: G equals its transpose
    bit for bit, every entry of a bound check against the oracle, and for
    256 < d <= 768 it equals, bit for bit, the full product written by the
    same 16-query kernel in the unfused comparator (no symmetry used)."""
    C = synth.dense_case(1, n, d, "unit", key=31 * n + d)[1]
    Cd = T(C)
    G = vs.vs_diversity_gram(Cd)[:, :n]
    assert torch.equal(G, G.t())
    Gh = G.cpu().numpy()
    ref = oracle.gram_cos(C, threads=8)
    assert np.abs(Gh.astype(np.float64) - ref).max() <= 2e-6
    if 256 < d:
        S = torch.empty((n, (n + 63) // 64 * 64), dtype=torch.float32, device=dev())
        vs.vs_bmu_search_unfused(Cd, Cd, vs.VS_COS_MAX, S=S)
        assert torch.equal(G, S[:, :n])


def test_diversity_gram_invalid_reference():
    """A reference outside [0, n) yields -1, NaN and leaves the mask alone;
    a sequence with every row masked yields -1 and NaN."""
    C = synth.dense_case(1, 100, 8, "unit", key=3)[1]
    G = vs.vs_diversity_gram(T(C))
    last = T(np.array([5, -1, 100, 7], np.int32))
    m = seed_masks(100, [5, 0, 0, 7])
    m[3, :] = 0xFFFFFFFF
    mask = T(m.view(np.int32))
    before = mask.cpu().numpy().copy()
    idx, score = vs.vs_diversity_step_gram(G, last, mask)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    after = mask.cpu().numpy()
    assert idx[1] == -1 and idx[2] == -1 and idx[3] == -1
    assert np.isnan(score[1:]).all()
    assert idx[0] >= 0
    assert np.array_equal(after[1:], before[1:])


def test_diversity_walk():
    w = diversity_walk()
    picks, scores, masks = gpu_chain(w["C"], [w["seed"]], len(w["picks"]))
    assert list(picks[0]) == w["picks"]
    for got, exp in zip(scores[0], w["values"]):
        assert (np.isnan(got) and np.isnan(exp)) or abs(got - exp) <= 1e-6


@pytest.mark.parametrize("n,d,nseq,steps", [(40, 3, 5, 41), (300, 64, 129, 20),
                                            (1000, 65, 300, 12), (129, 768, 70, 6),
                                            (3000, 128, 300, 4), (2000, 768, 260, 3),
                                            (700, 500, 520, 5)])
def test_diversity_chain(n, d, nseq, steps, div_kernel):
    C = synth.dense_case(1, n, d, "unit", key=n + d)[1]
    (r,) = synth.rng_children(900 + n, 1)
    seeds = r.choice(n, nseq, replace=nseq > n).astype(np.int32)
    picks, scores, masks = gpu_chain(C, seeds, steps)
    fails, stats = validate_chain(C, seeds, picks, scores, masks)
    assert not fails, fails


def test_diversity_matches_direct_run(div_kernel):
    """Tie-free small case: the GPU chain equals the oracle's own greedy run."""
    C = synth.dense_case(1, 500, 32, "unit", key=4242)[1]
    seeds = np.arange(0, 500, 7, dtype=np.int32)
    picks, scores, _ = gpu_chain(C, seeds, 10)
    o_picks, o_vals = oracle.div_run(C, seeds, 10)
    assert np.array_equal(picks, o_picks)
    assert np.allclose(scores, o_vals, rtol=1e-4, atol=1e-6)


def test_diversity_invalid_reference(div_kernel):
    """A reference outside [0, n) yields -1 and leaves the mask alone."""
    C = synth.dense_case(1, 100, 8, "unit", key=3)[1]
    Cd = T(C)
    last = T(np.array([5, -1, 100, 7], np.int32))
    mask = T(seed_masks(100, [5, 0, 0, 7]).view(np.int32))
    before = mask.cpu().numpy().copy()
    idx, score = vs.vs_diversity_step(Cd, last, mask)
    idx = idx.cpu().numpy()
    after = mask.cpu().numpy()
    assert idx[1] == -1 and idx[2] == -1
    assert idx[0] >= 0 and idx[3] >= 0
    assert np.array_equal(after[1:3], before[1:3])


@pytest.mark.slow
def test_workload_3_gram_chain():
    """The full diversity workload from the cached Gram matrix: bit-identical
    to the per-step scan for all 64 steps of 3,584 sequences."""
    w = synth.workload(3)
    a = gpu_chain(w["C"], w["seeds"], w["steps"])
    b = gpu_chain_gram(w["C"], w["seeds"], w["steps"])
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2], b[2])


def test_workload_3_gram_run():
    """The full diversity workload as bench.py times it from the Gram matrix:
    one vs_diversity_run_gram launch for all 64 steps of 3,584 sequences
    (and the triangle Gram build) equals the per-step MFMA scan bit for bit:
    picks, scores and final masks."""
    w = synth.workload(3)
    a = gpu_chain(w["C"], w["seeds"], w["steps"])
    Cd = T(w["C"])
    n = w["C"].shape[0]
    G = vs.vs_diversity_gram(Cd)
    mask = T(seed_masks(n, w["seeds"]).view(np.int32))
    picks, scores = vs.vs_diversity_run_gram(G, T(np.asarray(w["seeds"], np.int32)), mask,
                                             w["steps"])
    torch.cuda.synchronize()
    assert np.array_equal(picks.cpu().numpy().T, a[0])
    assert np.array_equal(scores.cpu().numpy().T.view(np.uint32), a[1].view(np.uint32))
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), a[2])


def test_workload_3_gram_centroid_run():
    """The centroid reading at full size, as bench.py times it: one
    vs_diversity_run_gram launch with running sums equals the chained
    vs_diversity_step_gram_sum calls bit for bit (picks, scores, masks and
    the final running sums)."""
    w = synth.workload(3)
    Cd = T(w["C"])
    n, nseq, steps = w["C"].shape[0], len(w["seeds"]), w["steps"]
    seeds = T(np.asarray(w["seeds"], np.int32))
    G = vs.vs_diversity_gram(Cd)
    m1 = T(seed_masks(n, w["seeds"]).view(np.int32))
    R1 = vs.vs_diversity_gram_sums(G, nseq)
    p1 = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    s1 = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    last = seeds
    for t in range(steps):
        vs.vs_diversity_step_gram_sum(G, last, R1, m1, idx_out=p1[t], score_out=s1[t])
        last = p1[t]
    m2 = T(seed_masks(n, w["seeds"]).view(np.int32))
    R2 = vs.vs_diversity_gram_sums(G, nseq)
    p2, s2 = vs.vs_diversity_run_gram(G, seeds, m2, steps, R=R2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(m1, m2)
    assert torch.equal(R1, R2)


@pytest.mark.slow
def test_workload_3_full_chain():
    """8,359 x 768 table, 3,584 sequences, 64 steps, every pick replayed."""
    w = synth.workload(3)
    picks, scores, masks = gpu_chain(w["C"], w["seeds"], w["steps"])
    fails, stats = validate_chain(w["C"], w["seeds"], picks, scores, masks, threads=16)
    assert not fails, fails
    assert stats["rows"] == 3584 * 64


# ------------------------------------------------------------------ CSR --

def padded(CT, pad):
    """Device copy of CT whose rows are `pad` elements longer than nc (a view
    with row stride nc + pad, as a caller avoiding cache-set aliasing would
    allocate it)."""
    if pad == 0:
        return T(CT)
    buf = torch.empty((CT.shape[0], CT.shape[1] + pad), dtype=torch.float32, device=dev())
    view = buf[:, :CT.shape[1]]
    view.copy_(torch.from_numpy(CT).to(dev()))
    return view


def run_csr(indptr, indices, values, CT, metric, pad=0):
    idx, score = vs.vs_bmu_search_csr(T(indptr), T(indices), T(values), padded(CT, pad), metric)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), score.cpu().numpy()


def test_csr_hand_cases(chunk):
    CT, rows = csr_cases()
    for r in rows:
        indptr = np.array([0, len(r["idx"])], np.int32)
        idx, score = run_csr(indptr, np.array(r["idx"] or [0], np.int32)[:len(r["idx"])],
                             np.array(r["val"] or [0], np.float32)[:len(r["val"])], CT,
                             r["metric"])
        assert idx[0] == r["expect_idx"], r
        assert abs(score[0] - r["expect_value"]) <= 1e-6, r


@pytest.fixture(params=["32", "64"])
def chunk(request, monkeypatch):
    """Run with each CSR chunk width (32 neurons = two queries per wave, 64 =
    one query per wave); both must satisfy the same bar."""
    monkeypatch.setenv("VS_CSR_CHUNK", request.param)
    return request.param


def csr_case(nq, d, nc, p, key, empty_rows=()):
    (r,) = synth.rng_children(3000 + key, 1)
    indptr, indices, values = synth.sparse_rows(r, nq, d, p)
    for e in empty_rows:
        lo, hi = int(indptr[e]), int(indptr[e + 1])
        indices = np.concatenate([indices[:lo], indices[hi:]])
        values = np.concatenate([values[:lo], values[hi:]])
        indptr = indptr.copy()
        indptr[e + 1:] -= hi - lo
    CT = synth.uniform01(r, (d, nc))
    synth.normalize_columns(CT)
    return indptr, indices, values, CT


def csr_parity(indptr, indices, values, CT, metric, threads=8):
    idx, score = run_csr(indptr, indices, values, CT, metric)
    o_idx, o_val, o_gap = oracle.csr(indptr, indices, values, CT, metric, threads=threads)
    if metric in (0, 1):
        qn = np.array([np.sum(values[indptr[i]:indptr[i + 1]].astype(np.float64) ** 2)
                       for i in range(len(indptr) - 1)])
        floor = 1e-2 * (qn + 1.0)
    else:
        floor = 1e-2
    cscale = oracle.sqnorms(CT, feature_major=True)

    def pv(rows, cand):
        out = np.empty(rows.size)
        for t, (i, j) in enumerate(zip(rows, cand)):
            sub = np.array([0, indptr[i + 1] - indptr[i]], np.int32)
            ii = indices[indptr[i]:indptr[i + 1]]
            vv = values[indptr[i]:indptr[i + 1]]
            col = np.ascontiguousarray(CT[:, j:j + 1])
            _, v, _ = oracle.csr(sub, ii, vv, col, metric, col_sq=cscale[j:j + 1])
            out[t] = v[0]
        return out

    fails, stats = check(idx, score, o_idx, o_val, o_gap, metric, floor, pv)
    assert not fails, fails
    return stats


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
@pytest.mark.parametrize("nc", [1, 63, 256, 1000, 1028])
def test_csr_shapes(metric, nc, chunk):
    empty = () if metric in (2, 3) else (0, 5)
    indptr, indices, values, CT = csr_case(70, 300, nc, 0.05, key=nc * 4 + metric,
                                           empty_rows=empty)
    csr_parity(indptr, indices, values, CT, metric)


@pytest.mark.parametrize("metric", [0, 2])
def test_csr_wide_vocabulary(metric):
    """A 65,536-feature vocabulary (four times the sparse workload's): the
    codebook slices hold 64 neurons x 65,536 features, and the blocked copy
    agrees with the plain layout bit for bit."""
    indptr, indices, values, CT = csr_case(60, 65536, 300, 0.002, key=640 + metric)
    csr_parity(indptr, indices, values, CT, metric)
    a = run_csr(indptr, indices, values, CT, metric)
    b = run_csr_blocked(indptr, indices, values, CT, metric)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("pad", [1, 64])
def test_csr_row_stride(pad, chunk):
    """A padded codebook row stride (ldct > nc) gives bit-identical results."""
    indptr, indices, values, CT = csr_case(90, 200, 700, 0.05, key=55)
    a = run_csr(indptr, indices, values, CT, 0)
    b = run_csr(indptr, indices, values, CT, 0, pad=pad)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    csr_parity(indptr, indices, values, CT, 0)


@pytest.mark.parametrize("metric", [0, 2])
def test_csr_paths_agree_bitwise(metric, monkeypatch):
    """The four-rows-per-load kernel and the 4-byte-load kernels (one or two
    queries per wave) sum in the same order, so they agree bit for bit, on
    both codebook layouts."""
    indptr, indices, values, CT = csr_case(150, 300, 1030 - 1030 % 4, 0.06, key=66 + metric)
    outs = []
    for env in ({"VS_CSR_CHUNK": "64"}, {"VS_CSR_CHUNK": "64", "VS_CSR_DWORD": "1"},
                {"VS_CSR_CHUNK": "32"}):
        monkeypatch.delenv("VS_CSR_DWORD", raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        outs.append(run_csr(indptr, indices, values, CT, metric))
        outs.append(run_csr_blocked(indptr, indices, values, CT, metric))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0])
        assert np.array_equal(o[1].view(np.uint32), outs[0][1].view(np.uint32))


def run_csr_blocked(indptr, indices, values, CT, metric, pad=0):
    CB = vs.vs_csr_block_codebook(padded(CT, pad))
    idx, score = vs.vs_bmu_search_csr_blocked(T(indptr), T(indices), T(values), CB,
                                              CT.shape[1], metric, d=CT.shape[0])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), score.cpu().numpy()


@pytest.mark.parametrize("metric", [0, 3])
def test_csr_unsorted_rows(metric, chunk):
    """Column order inside a row is free (only uniqueness is required): rows
    whose entries are shuffled meet the oracle's bar, and the blocked layout
    still agrees with the plain one bit for bit."""
    indptr, indices, values, CT = csr_case(70, 300, 1000, 0.05, key=77 + metric)
    (r,) = synth.rng_children(3100 + metric, 1)
    ix, vv = indices.copy(), values.copy()
    for i in range(len(indptr) - 1):
        lo, hi = int(indptr[i]), int(indptr[i + 1])
        perm = r.permutation(hi - lo)
        ix[lo:hi] = indices[lo:hi][perm]
        vv[lo:hi] = values[lo:hi][perm]
    assert not np.array_equal(ix, indices)
    csr_parity(indptr, ix, vv, CT, metric)
    a = run_csr(indptr, ix, vv, CT, metric)
    b = run_csr_blocked(indptr, ix, vv, CT, metric)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("nc,pad", [(1, 0), (63, 0), (64, 0), (700, 3), (1030, 0), (1028, 64)])
def test_csr_block_codebook_layout(nc, pad):
    """The blocked copy holds feature k of neuron 64 b + j at (b d + k) 64 + j
    and zeros past nc (an exact copy, checked against numpy indexing)."""
    d = 37
    (r,) = synth.rng_children(4100 + nc, 1)
    CT = synth.uniform01(r, (d, nc))
    CB = vs.vs_csr_block_codebook(padded(CT, pad)).cpu().numpy()
    nb = (nc + 63) // 64
    exp = np.zeros((nb, d, 64), np.float32)
    for b in range(nb):
        w = min(64, nc - 64 * b)
        exp[b, :, :w] = CT[:, 64 * b:64 * b + w]
    assert CB.shape == (nb * d * 64,)
    assert np.array_equal(CB.reshape(nb, d, 64).view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
@pytest.mark.parametrize("nc", [1, 63, 700, 1028])
def test_csr_blocked_matches_plain(metric, nc, chunk):
    """The blocked layout is read by the same kernels in the same order:
    results are bit-identical to the plain feature-major search, which the
    oracle checks."""
    empty = () if metric in (2, 3) else (0, 5)
    indptr, indices, values, CT = csr_case(70, 300, nc, 0.05, key=nc * 8 + metric,
                                           empty_rows=empty)
    a = run_csr(indptr, indices, values, CT, metric)
    b = run_csr_blocked(indptr, indices, values, CT, metric)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    csr_parity(indptr, indices, values, CT, metric)


def run_csr_f16(indptr, indices, values, CT, metric, pad=0):
    CB16 = vs.vs_csr_block_codebook_f16(padded(CT, pad))
    idx, score = vs.vs_bmu_search_csr_blocked_f16(T(indptr), T(indices), T(values), CB16,
                                                  CT.shape[1], metric, d=CT.shape[0])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), score.cpu().numpy()


def f16_rounded(CT):
    """The codebook as the fp16 path stores it (IEEE binary16, nearest even),
    held in fp32 (exact)."""
    return CT.astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("nc", [1, 63, 100, 128, 300, 1030])
def test_csr_blocked_to_f16_equals_plain(nc):
    """The fp16 copy made from the 64-neuron blocked fp32 codebook equals,
    bit for bit, the one made from the plain feature-major codebook."""
    d = 41
    (r,) = synth.rng_children(4300 + nc, 1)
    CT = synth.uniform01(r, (d, nc))
    a = vs.vs_csr_block_codebook_f16(T(CT))
    b = vs.vs_csr_blocked_to_f16(vs.vs_csr_block_codebook(T(CT)), nc, d)
    torch.cuda.synchronize()
    assert a.numel() == b.numel()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("nc,pad", [(1, 0), (100, 0), (128, 0), (300, 5), (1030, 0)])
def test_csr_block_codebook_f16_layout(nc, pad):
    """The fp16 blocked copy holds fp16(feature k of neuron 128 b + j) at
    (b d + k) 128 + j and zeros past nc: numpy's float16 rounding (nearest
    even) bit for bit."""
    d = 29
    (r,) = synth.rng_children(4200 + nc, 1)
    CT = synth.normal(r, (d, nc), std=2.0)
    CB = vs.vs_csr_block_codebook_f16(padded(CT, pad)).cpu().numpy()
    nb = (nc + 127) // 128
    exp = np.zeros((nb, d, 128), np.float16)
    for b in range(nb):
        w = min(128, nc - 128 * b)
        exp[b, :, :w] = CT[:, 128 * b:128 * b + w].astype(np.float16)
    assert CB.shape == (nb * d * 128,)
    assert np.array_equal(CB.reshape(nb, d, 128).view(np.uint16), exp.view(np.uint16))


@pytest.mark.parametrize("metric", [0, 1, 2, 3])
@pytest.mark.parametrize("nc", [1, 100, 700, 1028])
def test_csr_f16_storage(metric, nc):
    """fp16 storage, fp32 arithmetic: bit-identical to the fp32 search over
    the fp16-rounded codebook, which the oracle checks."""
    empty = () if metric in (2, 3) else (0, 5)
    indptr, indices, values, CT = csr_case(70, 300, nc, 0.05, key=nc * 16 + metric,
                                           empty_rows=empty)
    CT16 = f16_rounded(CT)
    a = run_csr_f16(indptr, indices, values, CT, metric)
    b = run_csr(indptr, indices, values, CT16, metric)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    csr_parity(indptr, indices, values, CT16, metric)


def csr_select(indptr, indices, values, rows):
    rows = np.asarray(rows)
    ptr = np.concatenate([[0], np.cumsum(indptr[rows + 1] - indptr[rows])]).astype(np.int32)
    idx = np.concatenate([indices[indptr[i]:indptr[i + 1]] for i in rows]).astype(np.int32)
    val = np.concatenate([values[indptr[i]:indptr[i + 1]] for i in rows]).astype(np.float32)
    return ptr, idx, val


def test_csr_bad_rows_skipped(chunk):
    """A column index outside [0, d) makes its row report (-1, NaN); the
    other rows are unaffected."""
    indptr, indices, values, CT = csr_case(10, 50, 64, 0.2, key=77)
    bad = int(np.nonzero(indptr[1:] > indptr[:-1])[0][0])
    indices = indices.copy()
    indices[indptr[bad]] = 50  # == d
    idx, score = run_csr(indptr, indices, values, CT, 0)
    assert idx[bad] == -1 and np.isnan(score[bad])
    good = np.array([i for i in range(10) if i != bad])
    o_idx, _, _ = oracle.csr(*csr_select(indptr, indices, values, good), CT, 0)
    assert np.array_equal(idx[good], o_idx)


@pytest.mark.slow
def test_workload_4_seeded_rows():
    """32,768 CSR rows (~164 nnz of 16,384) x 65,536 neurons at full size;
    4,096 seeded rows are checked one by one against the oracle."""
    w = synth.workload(4)
    idx, score = run_csr(w["indptr"], w["indices"], w["values"], w["CT"], 0, pad=64)
    # the blocked layout (the form the benchmark times) gives the same bits
    bidx, bscore = run_csr_blocked(w["indptr"], w["indices"], w["values"], w["CT"], 0)
    assert np.array_equal(idx, bidx)
    assert np.array_equal(score.view(np.uint32), bscore.view(np.uint32))
    del bidx, bscore
    sel = synth.sample_queries(w["nq"], 4096, key=4)
    ptr = w["indptr"]
    sub_ptr = np.concatenate([[0], np.cumsum(ptr[sel + 1] - ptr[sel])]).astype(np.int32)
    sub_idx = np.concatenate([w["indices"][ptr[i]:ptr[i + 1]] for i in sel])
    sub_val = np.concatenate([w["values"][ptr[i]:ptr[i + 1]] for i in sel])
    col_sq = oracle.sqnorms(w["CT"], feature_major=True, threads=16)
    o_idx, o_val, o_gap = oracle.csr(sub_ptr, sub_idx, sub_val, w["CT"], 0, col_sq=col_sq,
                                     threads=16)
    qn = np.array([np.sum(sub_val[sub_ptr[i]:sub_ptr[i + 1]].astype(np.float64) ** 2)
                   for i in range(len(sel))])
    fails, stats = check(idx[sel], score[sel], o_idx, o_val, o_gap, 0, 1e-2 * (qn + 1.0),
                         lambda r, c: np.array([
                             oracle.csr(np.array([0, sub_ptr[i + 1] - sub_ptr[i]], np.int32),
                                        sub_idx[sub_ptr[i]:sub_ptr[i + 1]],
                                        sub_val[sub_ptr[i]:sub_ptr[i + 1]],
                                        np.ascontiguousarray(w["CT"][:, j:j + 1]), 0,
                                        col_sq=col_sq[j:j + 1])[1][0]
                             for i, j in zip(r, c)]))
    assert not fails, fails
    assert stats["rows"] == 4096 and stats["floor_bound"] == 0, stats
    assert (idx >= 0).all()
    print("workload 4 parity:", stats)


@pytest.mark.slow
def test_workload_4_f16_storage():
    """The full-size sparse workload with the codebook stored in fp16: equal,
    bit for bit, to the fp32 search over the fp16-rounded codebook, and 256
    seeded rows checked one by one against the oracle on that codebook."""
    w = synth.workload(4)
    CT16 = f16_rounded(w["CT"])
    idx, score = run_csr_f16(w["indptr"], w["indices"], w["values"], w["CT"], 0)
    ridx, rscore = run_csr(w["indptr"], w["indices"], w["values"], CT16, 0, pad=64)
    assert np.array_equal(idx, ridx)
    assert np.array_equal(score.view(np.uint32), rscore.view(np.uint32))
    sel = synth.sample_queries(w["nq"], 256, key=44)
    ptr = w["indptr"]
    sub_ptr = np.concatenate([[0], np.cumsum(ptr[sel + 1] - ptr[sel])]).astype(np.int32)
    sub_idx = np.concatenate([w["indices"][ptr[i]:ptr[i + 1]] for i in sel])
    sub_val = np.concatenate([w["values"][ptr[i]:ptr[i + 1]] for i in sel])
    col_sq = oracle.sqnorms(CT16, feature_major=True, threads=16)
    o_idx, o_val, o_gap = oracle.csr(sub_ptr, sub_idx, sub_val, CT16, 0, col_sq=col_sq,
                                     threads=16)
    qn = np.array([np.sum(sub_val[sub_ptr[i]:sub_ptr[i + 1]].astype(np.float64) ** 2)
                   for i in range(len(sel))])
    fails, stats = check(idx[sel], score[sel], o_idx, o_val, o_gap, 0, 1e-2 * (qn + 1.0),
                         lambda r, c: np.array([
                             oracle.csr(np.array([0, sub_ptr[i + 1] - sub_ptr[i]], np.int32),
                                        sub_idx[sub_ptr[i]:sub_ptr[i + 1]],
                                        sub_val[sub_ptr[i]:sub_ptr[i + 1]],
                                        np.ascontiguousarray(CT16[:, j:j + 1]), 0,
                                        col_sq=col_sq[j:j + 1])[1][0]
                             for i, j in zip(r, c)]))
    assert not fails, fails
