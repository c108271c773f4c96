"""GPU parity past 2^31 elements: a candidate table, a query set and a
diversity table each holding more than 2^31 floats (8 GiB and more), so
the rows at the end of each are reached only through 64-bit offsets.

The large arrays are built on the device from host blocks: a base block
repeated K times, then a tail block of distinct rows that lies wholly past
element 2^31 (in the diversity table so do the last 12,421 rows of the
repeated block).  Repeated rows tie exactly, and ties go to the lowest
index, so the answer over the whole array equals the oracle's answer over
the compressed array [base; tail], with compressed index j < B standing for
row j (the first copy) and B + t for tail row t.  The oracle computes that
answer in full; the GPU's picks must in addition be first copies.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check, l2_floor

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import farthest_vector_search_amd as vs  # noqa: E402

BIG = 2 ** 31  # elements


def dev():
    return torch.device("cuda:0")


@pytest.fixture(params=["qreg", "q16", "tiled"])
def kernel(request, monkeypatch):
    monkeypatch.setenv("VS_DENSE_KERNEL", request.param)
    return request.param


@pytest.fixture(params=["q16", "tiled"])
def div_kernel(request, monkeypatch):
    monkeypatch.setenv("VS_DIV_KERNEL", request.param)
    return request.param


def repeated(base, K, tail):
    """Device array [base x K; tail] (row-major, contiguous)."""
    B, d = base.shape
    out = torch.empty((K * B + tail.shape[0], d), dtype=torch.float32, device=dev())
    b = torch.from_numpy(np.ascontiguousarray(base)).to(dev())
    out[: K * B].view(K, B, d).copy_(b.unsqueeze(0).expand(K, B, d))
    out[K * B:].copy_(torch.from_numpy(np.ascontiguousarray(tail)).to(dev()))
    del b
    return out


def to_compressed(j, B, K):
    """Row index of the repeated array -> compressed index (first copies
    map to themselves, tail rows follow the base block)."""
    j = np.asarray(j).astype(np.int64)
    return np.where(j < K * B, j % B, B + (j - K * B))


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_candidates_past_2_31(kernel, threads):
    """Squared-L2 search of 512 queries against 8,392,704 candidates of
    d = 256 (the 4,096 tail rows start at element 2^31 exactly): queries
    near tail rows, near base rows, and unrelated ones."""
    d, B, K, T = 256, 65536, 128, 4096
    _, Cc = synth.dense_case(1, B + T, d, "normal", key=900)
    base, tail = Cc[:B], Cc[B:]
    assert K * B * d == BIG
    (r,) = synth.rng_children(901, 1)
    near_tail = Cc[B + np.linspace(0, T - 1, 256).astype(np.int64)]
    near_base = Cc[np.linspace(0, B - 1, 128).astype(np.int64)]
    Q = np.concatenate([near_tail + synth.normal(r, near_tail.shape, 0.3),
                        near_base + synth.normal(r, near_base.shape, 0.3),
                        synth.normal(r, (128, d))]).astype(np.float32)
    C = repeated(base, K, tail)
    idx, score = vs.vs_bmu_search(torch.from_numpy(Q).to(dev()), C, 0)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    del C
    release()
    # ties among copies: a base pick must be the first copy
    assert ((idx >= K * B) | (idx < B)).all()
    o_idx, o_val, o_gap = oracle.dense(Q, Cc, 0, threads=threads)
    fails, stats = check(to_compressed(idx, B, K), score, o_idx, o_val, o_gap, 0,
                         l2_floor(Q, Cc, o_idx),
                         lambda rr, cc: oracle.pair_values(Q, Cc, 0, rr, cc))
    assert not fails, fails
    assert stats["rows"] == 512 and stats["floor_bound"] == 0, stats
    assert (idx[:256] >= K * B).all()  # the planted tail answers were found


def test_queries_past_2_31(kernel, threads):
    """8,392,704 queries of d = 256 (the 4,096 tail rows start at element
    2^31) against 4,096 candidates: the first copy of the base block and the
    tail are checked against the oracle, every other copy must return the
    first copy's answer bit for bit."""
    d, B, K, T = 256, 65536, 128, 4096
    Qc, C = synth.dense_case(B + T, 4096, d, "normal", key=902)
    C = (0.5 * C).astype(np.float32)
    Q = repeated(Qc[:B], K, Qc[B:])
    idx, score = vs.vs_bmu_search(Q, torch.from_numpy(C).to(dev()), 0)
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    del Q
    release()
    rows = np.concatenate([np.arange(B), K * B + np.arange(T)])
    o_idx, o_val, o_gap = oracle.dense(Qc, C, 0, threads=threads)
    fails, stats = check(idx[rows], score[rows], o_idx, o_val, o_gap, 0, l2_floor(Qc, C, o_idx),
                         lambda rr, cc: oracle.pair_values(Qc, C, 0, rr, cc))
    assert not fails, fails
    assert stats["rows"] == B + T and stats["floor_bound"] == 0, stats
    copies_i = idx[: K * B].reshape(K, B)
    copies_s = score[: K * B].view(np.uint32).reshape(K, B)
    assert (copies_i == copies_i[0]).all() and (copies_s == copies_s[0]).all()


def test_diversity_table_past_2_31(div_kernel, threads):
    """One diversity step over a table of 2,812,720 unit rows of d = 768
    (the 8,359 x 768 workload table repeated 336 times, then 4,096 distinct
    rows; the last 16,517 rows lie past element 2^31), for 64 sequences whose
    last picks lie past that bound: 32 in the tail, 32 in the last copies of
    the table.  The seed's other copies are never the answer (cosine 1 is
    the largest), so the compressed table gives the exact answer."""
    base = synth.workload(3)["C"]
    B, d = base.shape
    K, T = 336, 4096
    (rt, rs) = synth.rng_children(903, 2)
    tail = synth.normalize_rows(synth.normal(rt, (T, d)))
    n = K * B + T
    first_past = -(-BIG // d)  # first row that starts past element 2^31
    assert n * d > BIG and first_past < K * B
    seeds = np.concatenate([K * B + rs.choice(T, 32, replace=False),
                            rs.choice(np.arange(first_past, K * B), 32, replace=False)])
    seeds = seeds.astype(np.int32)
    nseq = len(seeds)
    W = (n + 31) // 32
    mask = np.zeros((nseq, W), np.uint32)
    mask[np.arange(nseq), seeds // 32] |= (np.uint32(1) << (seeds % 32).astype(np.uint32))
    C = repeated(base, K, tail)
    md = torch.from_numpy(mask.view(np.int32)).to(dev())
    idx, score = vs.vs_diversity_step(C, torch.from_numpy(seeds).to(dev()), md)
    idx, score, md = idx.cpu().numpy(), score.cpu().numpy(), md.cpu().numpy().view(np.uint32)
    del C
    release()
    assert ((idx >= K * B) | (idx < B)).all()  # first copies only
    Cc = np.concatenate([base, tail])
    sc = to_compressed(seeds, B, K)
    Wc = (Cc.shape[0] + 31) // 32
    mc = np.zeros((nseq, Wc), np.uint32)
    mc[np.arange(nseq), sc // 32] |= (np.uint32(1) << (sc % 32).astype(np.uint32))
    o_idx, o_val, o_gap = oracle.dense(Cc[sc], Cc, 3, mask=mc, threads=threads)
    fails, stats = check(to_compressed(idx, B, K), score, o_idx, o_val, o_gap, 3, 1e-2,
                         lambda rr, cc: oracle.pair_values(Cc[sc], Cc, 3, rr, cc))
    assert not fails, fails
    assert stats["rows"] == nseq and stats["empty"] == 0, stats
    # each mask row: the seed's bit and the pick's bit, nothing else
    exp = mask.copy()
    exp[np.arange(nseq), idx // 32] |= (np.uint32(1) << (idx % 32).astype(np.uint32))
    assert np.array_equal(md, exp)
    assert (np.unpackbits(md.view(np.uint8), axis=1).sum(axis=1) == 2).all()


def test_sparse_codebook_past_2_31(threads):
    """CSR search over a feature-major codebook of 8,192 features x 266,240
    neurons (2.18e9 floats: a 4,096-neuron base block repeated 64 times, then
    4,096 distinct neurons).  In the plain layout the features from 8,066 on
    lie past element 2^31 for every neuron (64 of the 512 queries draw all
    their non-zeros there); in the 64-neuron blocked copy the distinct tail
    does.  Both layouts must give the same bits and the oracle's answer over
    the compressed codebook."""
    d, B, K, T = 8192, 4096, 64, 4096
    nc = K * B + T
    k_hi = -(-BIG // nc)  # first feature row that starts past element 2^31
    assert d * nc > BIG and k_hi < d
    rq, rh, rc = synth.rng_children(904, 3)
    ip1, ix1, v1 = synth.sparse_rows(rq, 448, d, 164.0 / d)
    ip2, ix2, v2 = synth.sparse_rows(rh, 64, d - k_hi, 0.25)
    indptr = np.concatenate([ip1, ip2[1:] + ip1[-1]]).astype(np.int32)
    indices = np.concatenate([ix1, ix2 + k_hi]).astype(np.int32)
    values = np.concatenate([v1, v2]).astype(np.float32)
    CTc = synth.uniform01(rc, (d, B + T))
    synth.normalize_columns(CTc)
    CT = torch.empty((d, nc), dtype=torch.float32, device=dev())
    base = torch.from_numpy(np.ascontiguousarray(CTc[:, :B])).to(dev())
    CT[:, : K * B].view(d, K, B).copy_(base.unsqueeze(1).expand(d, K, B))
    CT[:, K * B:].copy_(torch.from_numpy(np.ascontiguousarray(CTc[:, B:])).to(dev()))
    del base
    Tq = [torch.from_numpy(a).to(dev()) for a in (indptr, indices, values)]
    a_idx, a_score = vs.vs_bmu_search_csr(*Tq, CT, 0)
    CB = vs.vs_csr_block_codebook(CT)
    del CT
    b_idx, b_score = vs.vs_bmu_search_csr_blocked(*Tq, CB, nc, 0, d=d)
    a_idx, a_score = a_idx.cpu().numpy(), a_score.cpu().numpy()
    b_idx, b_score = b_idx.cpu().numpy(), b_score.cpu().numpy()
    del CB
    release()
    assert np.array_equal(a_idx, b_idx)
    assert np.array_equal(a_score.view(np.uint32), b_score.view(np.uint32))
    assert ((a_idx >= K * B) | (a_idx < B)).all()  # first copies only
    o_idx, o_val, o_gap = oracle.csr(indptr, indices, values, CTc, 0, threads=threads)
    qn = np.array([np.sum(values[indptr[i]:indptr[i + 1]].astype(np.float64) ** 2)
                   for i in range(len(indptr) - 1)])
    cscale = oracle.sqnorms(CTc, feature_major=True)

    def pv(rows, cand):
        out = np.empty(rows.size)
        for t, (i, j) in enumerate(zip(rows, cand)):
            sub = np.array([0, indptr[i + 1] - indptr[i]], np.int32)
            col = np.ascontiguousarray(CTc[:, j:j + 1])
            _, v, _ = oracle.csr(sub, indices[indptr[i]:indptr[i + 1]],
                                 values[indptr[i]:indptr[i + 1]], col, 0, col_sq=cscale[j:j + 1])
            out[t] = v[0]
        return out

    fails, stats = check(to_compressed(a_idx, B, K), a_score, o_idx, o_val, o_gap, 0,
                         1e-2 * (qn + 1.0), pv)
    assert not fails, fails
    assert stats["rows"] == 512 and stats["floor_bound"] == 0, stats
