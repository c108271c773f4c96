"""vs_bmu_search_noalloc: the dense search with the library's own device
scratch array as its workspace (for callers that cannot allocate).

Called through the C ABI (ctypes, caller-allocated inputs and outputs, the
current torch stream) and compared with vs_bmu_search: the same kernels, so
the outputs must be identical bit for bit, and both must meet the oracle bar
(tests/parity.py).  Two calls in a row, the second on a smaller input, show
that what the first call left in the shared array does not leak into the
second.  Sizes beyond the array are refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from parity import check, l2_floor

torch = pytest.importorskip("torch")

import farthest_vector_search_amd as vs  # noqa: E402

SCRATCH_BYTES = 8 << 20
FAKE = 0x10000  # 256-byte aligned, never dereferenced by argument checks


def _P(x):
    return ctypes.c_void_p(x)


def _up(x):
    return (x + 255) // 256 * 256


def test_noalloc_validation():
    """Host-side checks only (no GPU needed): every refusal happens before
    anything is enqueued."""
    L = vs.lib()

    def call(Q=FAKE, C=FAKE, nq=4, nc=8, d=4, metric=0, idx=FAKE, score=FAKE):
        return L.vs_bmu_search_noalloc(_P(Q), _P(C), nq, nc, d, metric, _P(idx), _P(score),
                                       None)
    assert call(metric=4) == 3
    assert call(nq=-1) == 2
    assert call(nc=0) == 2
    assert call(d=0) == 2
    assert call(nq=0, Q=0, C=0, idx=0) == 0
    assert call(Q=0) == 1
    assert call(idx=0) == 1
    assert call(Q=FAKE + 2) == 5
    # the largest squared-L2 candidate count that fits beside 65,536 queries,
    # and one more 256-byte unit of candidates
    nq = 65536
    room = SCRATCH_BYTES - _up(8 * nq) - _up(4 * nq)
    assert L.vs_bmu_search_workspace(nq, room // 4, 256, 0) == SCRATCH_BYTES
    assert call(nq=nq, nc=room // 4 + 64, d=256) == 4
    # cosine metrics need only the keys
    assert call(nq=SCRATCH_BYTES // 8 + 32, nc=8, metric=2) == 4


def _dev():
    return torch.device("cuda:0")


def _noalloc(Q, C, metric, idx, score):
    rc = vs.lib().vs_bmu_search_noalloc(
        _P(Q.data_ptr()), _P(C.data_ptr()), Q.shape[0], C.shape[0], Q.shape[1], metric,
        _P(idx.data_ptr()), _P(score.data_ptr()),
        _P(torch.cuda.current_stream(_dev()).cuda_stream))
    assert rc == 0, vs.lib().vs_status_str(rc)


def _with_workspace(Q, C, metric):
    L = vs.lib()
    nq, d = Q.shape
    nc = C.shape[0]
    ws = torch.empty(max(L.vs_bmu_search_workspace(nq, nc, d, metric), 256), dtype=torch.uint8,
                     device=_dev())
    idx = torch.empty(nq, dtype=torch.int32, device=_dev())
    score = torch.empty(nq, dtype=torch.float32, device=_dev())
    rc = L.vs_bmu_search(_P(Q.data_ptr()), _P(C.data_ptr()), nq, nc, d, metric,
                         _P(idx.data_ptr()), _P(score.data_ptr()), _P(ws.data_ptr()),
                         ws.numel(), _P(torch.cuda.current_stream(_dev()).cuda_stream))
    assert rc == 0, L.vs_status_str(rc)
    return idx, score


@pytest.mark.gpu
@pytest.mark.parametrize("metric", [0, 2])
def test_noalloc_matches_workspace_search(metric):
    """Two calls in a row on the shared array, the second smaller, each
    compared bit for bit with vs_bmu_search and with the oracle."""
    dist = "unit" if metric in (2, 3) else "normal"
    shapes = [(3000, 5000, 64, 11), (300, 700, 33, 12), (256, 1024, 64, 13)]
    for nq, nc, d, key in shapes:
        print(f"noalloc metric {metric} nq {nq} nc {nc} d {d}", flush=True)
        Qn, Cn = synth.dense_case(nq, nc, d, dist, key=key)
        Q = torch.from_numpy(Qn).to(_dev())
        C = torch.from_numpy(Cn).to(_dev())
        # outputs pre-filled with garbage: every entry must be written
        idx = torch.full((nq,), -7, dtype=torch.int32, device=_dev())
        score = torch.full((nq,), 123.0, dtype=torch.float32, device=_dev())
        _noalloc(Q, C, metric, idx, score)
        ridx, rscore = _with_workspace(Q, C, metric)
        torch.cuda.synchronize()
        idx, score = idx.cpu().numpy(), score.cpu().numpy()
        assert np.array_equal(idx, ridx.cpu().numpy())
        assert np.array_equal(score.view(np.uint32), rscore.cpu().numpy().view(np.uint32))
        o_idx, o_val, o_gap = oracle.dense(Qn, Cn, metric, threads=8)
        floor = l2_floor(Qn, Cn, o_idx) if metric in (0, 1) else 1e-2
        fails, stats = check(idx, score, o_idx, o_val, o_gap, metric, floor,
                             lambda r, c: oracle.pair_values(Qn, Cn, metric, r, c))
        assert not fails, fails
        assert stats["rows"] == nq


@pytest.mark.gpu
def test_noalloc_at_its_size_limit():
    """A search whose workspace is exactly the array's 8 MiB: the 65,536 x
    16,384 workload's queries against 1,900,544 candidates would fill it; here
    a narrow version of the same layout (65,536 queries, as many candidates
    as fit, d = 4) against vs_bmu_search."""
    L = vs.lib()
    nq = 65536
    nc = (SCRATCH_BYTES - _up(8 * nq) - _up(4 * nq)) // 4
    assert L.vs_bmu_search_workspace(nq, nc, 4, 0) == SCRATCH_BYTES
    print(f"noalloc at limit nq {nq} nc {nc} d 4", flush=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    Q = torch.randn((nq, 4), generator=g).to(_dev())
    C = torch.randn((nc, 4), generator=g).to(_dev())
    idx = torch.empty(nq, dtype=torch.int32, device=_dev())
    score = torch.empty(nq, dtype=torch.float32, device=_dev())
    _noalloc(Q, C, 0, idx, score)
    ridx, rscore = _with_workspace(Q, C, 0)
    torch.cuda.synchronize()
    assert torch.equal(idx, ridx)
    assert torch.equal(score.view(torch.int32), rscore.view(torch.int32))


@pytest.mark.gpu
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("nq,nc", [(600, 3000), (256, 1024)])
def test_search_replays_from_a_captured_graph(entry, nq, nc):
    """The search captured into a HIP graph (three kernels, two for a small
    search; no memset node): every replay, with eager work and
    synchronisations between replays and different query contents each
    time, equals the eager search of the same contents bit for bit."""
    Qn, Cn = synth.dense_case(nq, nc, 64, "normal", key=21)
    Q = torch.from_numpy(Qn).to(_dev())
    C = torch.from_numpy(Cn).to(_dev())
    idx = torch.empty(nq, dtype=torch.int32, device=_dev())
    score = torch.empty(nq, dtype=torch.float32, device=_dev())
    L = vs.lib()
    ws = torch.empty(L.vs_bmu_search_workspace(nq, nc, 64, 0), dtype=torch.uint8, device=_dev())

    def call():
        if entry == "noalloc":
            _noalloc(Q, C, 0, idx, score)
        else:
            vs.vs_bmu_search(Q, C, 0, idx_out=idx, score_out=score, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # first call on the device outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        Q.copy_(torch.from_numpy(Qn * np.float32(1 + rep)).to(_dev()))
        g.replay()
        torch.cuda.synchronize()
        got_i, got_s = idx.clone(), score.clone()
        idx.fill_(-5)
        call()  # eager, same contents
        torch.cuda.synchronize()
        assert torch.equal(got_i, idx), rep
        assert torch.equal(got_s.view(torch.int32), score.view(torch.int32)), rep
