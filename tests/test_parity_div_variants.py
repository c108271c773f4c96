"""GPU parity of the diversity variants: the centroid reference and
full-length runs (through the C ABI).

"Issue 9-014: Tile Diversity Shader Inner Loop For L2 Cache Locality":
each step takes the unmasked candidate most different from the reference
and masks it ("Current Behavior"); "FP16 storage (compounding optimization)"
ranks against the sequence's centroid.  The GPU keeps, per sequence, the fp32
sum of its rows (vs_diversity_accumulate) and ranks by the dot product with
it (vs_diversity_step_ref); the oracle replays every recorded step from its
own prefix with the fp64 centroid and the true cosine.  Bar: as the other
diversity tests (tests/parity.py), on the cosine: the GPU's cosine is its
score divided by the norm of its reference row at that step.

Full-length runs take every row of the table (n - 1 picks after the seed)
and then report -1; the Gram step skips the loads of fully masked columns.
"""
import numpy as np
import pytest

import oracle
import synth
from goldens import diversity_centroid
from parity import check
from test_parity_div_csr import (T, dev, gpu_chain, gpu_chain_gram, seed_masks,  # noqa: F401
                                 validate_chain, div_kernel)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import farthest_vector_search_amd as vs  # noqa: E402


def gpu_chain_centroid(C, seeds, steps):
    """Centroid-reference run on the GPU: returns picks, cosines (score over
    the reference norm at that step), final masks and the final sums."""
    Cd = T(C)
    nseq = len(seeds)
    seeds_d = T(np.asarray(seeds, np.int32)).long()
    Q = Cd[seeds_d].contiguous()
    mask = T(seed_masks(C.shape[0], seeds).view(np.int32))
    picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    scores = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    norms = torch.empty((steps, nseq), dtype=torch.float64, device=dev())
    ws = torch.empty(vs.lib().vs_diversity_step_workspace(C.shape[0], C.shape[1], nseq),
                     dtype=torch.uint8, device=dev())
    for t in range(steps):
        norms[t] = torch.linalg.vector_norm(Q.double(), dim=1)
        vs.vs_diversity_step_ref(Cd, Q, mask, idx_out=picks[t], score_out=scores[t], workspace=ws)
        vs.vs_diversity_accumulate(Cd, picks[t], Q)
    torch.cuda.synchronize()
    picks = picks.cpu().numpy().T.copy()
    cos = (scores.double() / norms).cpu().numpy().T.copy()
    cos[picks < 0] = np.nan
    return picks, cos, mask.cpu().numpy().view(np.uint32), Q.cpu().numpy()


def validate_centroid(C, seeds, picks, cos, masks, threads=8):
    rep = oracle.div_replay_centroid(C, seeds, picks, threads=threads)
    fails = []
    live = rep["bidx"] >= 0
    if not (rep["pick_ok"][live] == 1).all():
        fails.append("illegal pick (masked or out of range)")
    if not (picks[~live] == -1).all():
        fails.append("pick where nothing was left")
    f, stats = check(picks.reshape(-1), cos.reshape(-1), rep["bidx"].reshape(-1),
                     rep["best"].reshape(-1), rep["gap"].reshape(-1), 3, 1e-2,
                     lambda r, c: rep["pick_value"].reshape(-1)[r],
                     legal=lambda r, c: rep["pick_ok"].reshape(-1)[r] == 1)
    fails += f
    exp = seed_masks(C.shape[0], seeds)
    for s in range(picks.shape[0]):
        for p in picks[s]:
            if p >= 0:
                exp[s, p // 32] |= np.uint32(1 << (p % 32))
    if not np.array_equal(exp, masks):
        fails.append("final masks differ from seed + picks")
    return fails, stats


# ----------------------------------------------------------- centroid --

def test_centroid_walk():
    """The hand-worked plane walk (tests/golden/diversity_centroid.txt)."""
    w = diversity_centroid()
    picks, cos, _, _ = gpu_chain_centroid(w["C"], np.array([w["seed"]], np.int32),
                                          len(w["picks"]))
    assert list(picks[0]) == w["picks"]
    for v, e in zip(cos[0], w["values"]):
        assert (np.isnan(v) and np.isnan(e)) or abs(v - e) <= 1e-6


@pytest.mark.parametrize("n,d,nseq,steps", [(40, 3, 5, 41), (300, 64, 129, 20),
                                            (1000, 65, 300, 12), (129, 768, 70, 6),
                                            (700, 500, 520, 5)])
def test_centroid_chain(n, d, nseq, steps, div_kernel):
    C = synth.dense_case(1, n, d, "unit", key=n + d + 1)[1]
    (r,) = synth.rng_children(1900 + n, 1)
    seeds = r.choice(n, nseq, replace=nseq > n).astype(np.int32)
    picks, cos, masks, _ = gpu_chain_centroid(C, seeds, steps)
    fails, _ = validate_centroid(C, seeds, picks, cos, masks)
    assert not fails, fails


def test_centroid_matches_direct_run(div_kernel):
    """Tie-free small case: the GPU run equals the oracle's own run."""
    C = synth.dense_case(1, 500, 32, "unit", key=4343)[1]
    seeds = np.arange(3, 500, 9, dtype=np.int32)
    picks, cos, _, _ = gpu_chain_centroid(C, seeds, 12)
    o_picks, o_vals = oracle.div_run_centroid(C, seeds, 12, threads=8)
    assert np.array_equal(picks, o_picks)
    assert np.allclose(cos, o_vals, rtol=1e-4, atol=1e-6)


def test_reference_step_equals_gathered_step(div_kernel):
    """With Q = C[last] the explicit-reference step is the gathered step:
    same arithmetic, so picks, scores and masks agree bit for bit."""
    n, d, nseq = 900, 128, 200
    C = synth.dense_case(1, n, d, "unit", key=77)[1]
    (r,) = synth.rng_children(1977, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    Cd = T(C)
    m1 = T(seed_masks(n, seeds).view(np.int32))
    m2 = m1.clone()
    i1, s1 = vs.vs_diversity_step(Cd, T(seeds), m1)
    i2, s2 = vs.vs_diversity_step_ref(Cd, Cd[T(seeds).long()].contiguous(), m2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(m1, m2)


def test_accumulate_exact():
    """Q[s] + C[pick[s]] is one fp32 addition per element (numpy's); picks
    outside [0, n) leave their row alone."""
    n, d = 50, 37
    C = synth.dense_case(1, n, d, "normal", key=5)[1]
    Q0 = synth.dense_case(6, 1, d, "normal", key=6)[0]
    pick = np.array([3, -1, 49, 50, 0, 7], np.int32)
    Q = T(Q0)
    vs.vs_diversity_accumulate(T(C), T(pick), Q)
    got = Q.cpu().numpy()
    exp = Q0.copy()
    for s, p in enumerate(pick):
        if 0 <= p < n:
            exp[s] = Q0[s] + C[p]
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


@pytest.mark.slow
def test_workload_3_centroid():
    """8,359 x 768 table, 3,584 sequences, 64 centroid-reference steps; 96
    seeded sequences replayed step by step by the oracle."""
    w = synth.workload(3)
    picks, cos, masks, _ = gpu_chain_centroid(w["C"], w["seeds"], w["steps"])
    sel = synth.sample_queries(len(w["seeds"]), 96, key=3)
    fails, stats = validate_centroid(w["C"], w["seeds"][sel], picks[sel], cos[sel], masks[sel],
                                     threads=16)
    assert not fails, fails
    assert stats["rows"] == 96 * 64
    assert (picks >= 0).all()


# ------------------------------------------- centroid from the Gram matrix --

def gpu_chain_gram_centroid(C, seeds, steps):
    """Centroid-reference run from the cached Gram matrix: R[s] += G[last],
    masked arg-min of R[s].  Returns picks, cosines (score over the norm of
    the sum of the sequence's rows so far, taken on the host in fp64), masks."""
    Cd = T(C)
    nseq = len(seeds)
    mask = T(seed_masks(C.shape[0], seeds).view(np.int32))
    last = T(np.asarray(seeds, np.int32))
    picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    scores = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    G = vs.vs_diversity_gram(Cd)
    R = vs.vs_diversity_gram_sums(G, nseq)
    for t in range(steps):
        vs.vs_diversity_step_gram_sum(G, last, R, mask, idx_out=picks[t], score_out=scores[t])
        last = picks[t]
    torch.cuda.synchronize()
    picks = picks.cpu().numpy().T.copy()
    scores = scores.cpu().numpy().T.astype(np.float64)
    C64 = C.astype(np.float64)
    ref = C64[np.asarray(seeds)].copy()
    cos = np.full(picks.shape, np.nan)
    for t in range(steps):
        live = picks[:, t] >= 0
        cos[live, t] = scores[live, t] / np.linalg.norm(ref[live], axis=1)
        ref[live] += C64[picks[live, t]]
    return picks, cos, mask.cpu().numpy().view(np.uint32)


def test_gram_centroid_walk():
    """The hand-worked plane walk, the vectors padded with zeros to d = 4
    (cosines unchanged)."""
    w = diversity_centroid()
    C = np.zeros((w["C"].shape[0], 4), np.float32)
    C[:, :2] = w["C"]
    picks, cos, _ = gpu_chain_gram_centroid(C, np.array([w["seed"]], np.int32), len(w["picks"]))
    assert list(picks[0]) == w["picks"]
    for v, e in zip(cos[0], w["values"]):
        assert (np.isnan(v) and np.isnan(e)) or abs(v - e) <= 1e-6


@pytest.mark.parametrize("n,d,nseq,steps", [(40, 4, 5, 41), (300, 64, 129, 20),
                                            (129, 768, 70, 6), (700, 500, 520, 5)])
def test_gram_centroid_chain(n, d, nseq, steps):
    C = synth.dense_case(1, n, d, "unit", key=n + d + 1)[1]
    (r,) = synth.rng_children(1900 + n, 1)
    seeds = r.choice(n, nseq, replace=nseq > n).astype(np.int32)
    picks, cos, masks = gpu_chain_gram_centroid(C, seeds, steps)
    fails, _ = validate_centroid(C, seeds, picks, cos, masks)
    assert not fails, fails


def test_gram_centroid_full_length():
    n, d, nseq = 160, 48, 24
    C = synth.dense_case(1, n, d, "unit", key=888)[1]
    (r,) = synth.rng_children(2888, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    picks, cos, masks = gpu_chain_gram_centroid(C, seeds, n + 1)
    fails, _ = validate_centroid(C, seeds, picks, cos, masks)
    assert not fails, fails
    assert (picks[:, :n - 1] >= 0).all() and (picks[:, n - 1:] == -1).all()


def test_gram_centroid_invalid_reference():
    """A reference outside [0, n) gives -1 and leaves the mask and R alone."""
    C = synth.dense_case(1, 100, 8, "unit", key=3)[1]
    Cd = T(C)
    G = vs.vs_diversity_gram(Cd)
    R = vs.vs_diversity_gram_sums(G, 3)
    last = T(np.array([5, -1, 100], np.int32))
    mask = T(seed_masks(100, [5, 0, 0]).view(np.int32))
    before = mask.cpu().numpy().copy()
    idx, _ = vs.vs_diversity_step_gram_sum(G, last, R, mask)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    assert idx[0] >= 0 and idx[1] == -1 and idx[2] == -1
    assert np.array_equal(mask.cpu().numpy()[1:], before[1:])
    assert not R[1:].any()


@pytest.mark.slow
def test_workload_3_gram_centroid():
    """8,359 x 768 table, 3,584 sequences, 64 centroid-reference steps from the
    Gram matrix; 96 seeded sequences replayed by the oracle."""
    w = synth.workload(3)
    picks, cos, masks = gpu_chain_gram_centroid(w["C"], w["seeds"], w["steps"])
    sel = synth.sample_queries(len(w["seeds"]), 96, key=33)
    fails, stats = validate_centroid(w["C"], w["seeds"][sel], picks[sel], cos[sel], masks[sel],
                                     threads=16)
    assert not fails, fails
    assert (picks >= 0).all()


# --------------------------------------------------------- full length --

@pytest.mark.parametrize("n,d,nseq", [(300, 64, 40), (97, 8, 33)])
def test_full_length_last_pick(n, d, nseq, div_kernel):
    """Every row is taken once (n - 1 picks after the seed), then -1; both
    step kernels and the Gram step replay against the oracle, and the Gram
    step (built by the 16-query kernel's arithmetic) equals that kernel's
    per-step scan bit for bit."""
    C = synth.dense_case(1, n, d, "unit", key=n * 3 + d)[1]
    (r,) = synth.rng_children(2900 + n, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    steps = n + 2
    picks, scores, masks = gpu_chain(C, seeds, steps)
    fails, _ = validate_chain(C, seeds, picks, scores, masks)
    assert not fails, fails
    assert (picks[:, :n - 1] >= 0).all() and (picks[:, n - 1:] == -1).all()
    assert (masks[:, :n // 32] == 0xFFFFFFFF).all()
    g = gpu_chain_gram(C, seeds, steps)
    if div_kernel == "q16":
        assert np.array_equal(g[0], picks)
        assert np.array_equal(g[1].view(np.uint32), scores.view(np.uint32))
        assert np.array_equal(g[2], masks)
    else:
        fails, _ = validate_chain(C, seeds, *g)
        assert not fails, fails


def test_full_length_centroid(div_kernel):
    n, d, nseq = 160, 48, 24
    C = synth.dense_case(1, n, d, "unit", key=888)[1]
    (r,) = synth.rng_children(2888, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    picks, cos, masks, _ = gpu_chain_centroid(C, seeds, n + 1)
    fails, _ = validate_centroid(C, seeds, picks, cos, masks)
    assert not fails, fails
    assert (picks[:, :n - 1] >= 0).all() and (picks[:, n - 1:] == -1).all()


@pytest.mark.slow
def test_workload_3_full_length_gram():
    """All 8,358 picks of all 3,584 sequences from the cached Gram matrix; 16
    seeded sequences replayed over the whole run by the oracle."""
    w = synth.workload(3)
    n = w["C"].shape[0]
    picks, scores, masks = gpu_chain_gram(w["C"], w["seeds"], n - 1)
    assert (picks >= 0).all()
    assert all(len(np.unique(p)) == n - 1 for p in picks[:64])
    sel = synth.sample_queries(len(w["seeds"]), 16, key=31)
    fails, stats = validate_chain(w["C"], w["seeds"][sel], picks[sel], scores[sel], masks[sel],
                                  threads=16)
    assert not fails, fails
    assert stats["rows"] == 16 * (n - 1)


# ------------------------------------------------------------ whole runs --

@pytest.mark.parametrize("n,d,nseq,steps", [(300, 64, 129, 20), (1000, 65, 70, 9)])
def test_run_matches_steps(n, d, nseq, steps, div_kernel):
    """vs_diversity_run chains the steps on the stream: the same picks,
    scores and masks, bit for bit, as calling the step one by one."""
    C = synth.dense_case(1, n, d, "unit", key=n + 5 * d)[1]
    (r,) = synth.rng_children(2950 + n, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    p1, s1, m1 = gpu_chain(C, seeds, steps)
    mask = T(seed_masks(n, seeds).view(np.int32))
    p2, s2 = vs.vs_diversity_run(T(C), T(seeds), mask, steps)
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy().T, p1)
    assert np.array_equal(s2.cpu().numpy().T.view(np.uint32), s1.view(np.uint32))
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), m1)


def masks_for(n, seeds):
    """Seed masks; a seed outside [0, n) sets no bit."""
    W = (n + 31) // 32
    m = np.zeros((len(seeds), W), np.uint32)
    for s, j in enumerate(seeds):
        if 0 <= j < n:
            m[s, j // 32] |= np.uint32(1 << (j % 32))
    return m


# the whole-run kernel keeps a sequence's mask row in LDS up to 32,768 columns
# and falls back to per-step launches above; (n, d, nseq, steps, seeds)
RUN_GRAM_CASES = [
    (400, 96, 90, 30, "distinct"),
    (37, 8, 20, 40, "distinct"),       # exhausts every candidate, then -1
    (1, 4, 3, 3, "repeat"),            # nothing but the seed: -1 from the first step
    (2049, 16, 300, 12, "repeat"),     # sequences sharing a seed
    (777, 32, 40, 9, "invalid"),       # seeds -1 and n mixed in
    (32768, 4, 8, 3, "distinct"),      # widest mask row kept in LDS
    (32769, 4, 8, 3, "distinct"),      # one column more: per-step launches
]


@pytest.mark.parametrize("centroid", [False, True])
@pytest.mark.parametrize("n,d,nseq,steps,kind", RUN_GRAM_CASES)
def test_run_gram_matches_steps(centroid, n, d, nseq, steps, kind):
    """vs_diversity_run_gram (one launch per run where the mask row fits in
    LDS) equals the step-by-step calls bit for bit: picks, scores, masks and,
    for the centroid reading, the running sums of the live columns."""
    C = synth.dense_case(1, n, d, "unit", key=4000 + n + centroid)[1]
    (r,) = synth.rng_children(4100 + n, 1)
    if kind == "distinct":
        seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    else:
        seeds = r.choice(n, nseq, replace=True).astype(np.int32)
    if kind == "invalid":
        seeds[::7] = -1
        seeds[3::7] = n
    Cd = T(C)
    G = vs.vs_diversity_gram(Cd)
    # step by step
    m1 = T(masks_for(n, seeds).view(np.int32))
    R1 = vs.vs_diversity_gram_sums(G, nseq) if centroid else None
    p1 = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    s1 = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    last = T(seeds)
    for t in range(steps):
        if centroid:
            vs.vs_diversity_step_gram_sum(G, last, R1, m1, idx_out=p1[t], score_out=s1[t])
        else:
            vs.vs_diversity_step_gram(G, last, m1, idx_out=p1[t], score_out=s1[t])
        last = p1[t]
    # one call (R deliberately left dirty: the call clears it)
    m2 = T(masks_for(n, seeds).view(np.int32))
    R2 = None
    if centroid:
        R2 = vs.vs_diversity_gram_sums(G, nseq)
        R2.fill_(7.0)
    p2, s2 = vs.vs_diversity_run_gram(G, T(seeds), m2, steps, R=R2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(m1, m2)
    if centroid:
        # the sums are specified on live (unmasked) columns only
        bits = np.unpackbits(m2.cpu().numpy().view(np.uint8), bitorder="little",
                             axis=1)[:, :n].astype(bool)
        r1, r2 = R1.cpu().numpy(), R2.cpu().numpy()
        assert np.array_equal(r1.view(np.uint32)[~bits], r2.view(np.uint32)[~bits])
    p = p2.cpu().numpy()
    assert ((p >= 0) | (p == -1)).all()
    if kind == "invalid":
        bad = (seeds < 0) | (seeds >= n)
        assert (p[:, bad] == -1).all() and (p[:, ~bad][0] >= 0).all()
    if steps >= n:  # exhausted: n - 1 picks (a distinct seed each), then -1
        assert (p[n - 1:] == -1).all()


def test_run_ref_matches_steps(div_kernel):
    """vs_diversity_run_ref equals the step_ref / accumulate chain bit for bit."""
    n, d, nseq, steps = 500, 64, 100, 15
    C = synth.dense_case(1, n, d, "unit", key=4200)[1]
    (r,) = synth.rng_children(4201, 1)
    seeds = r.choice(n, nseq, replace=False).astype(np.int32)
    Cd = T(C)
    Q1 = Cd[T(seeds).long()].contiguous()
    m1 = T(seed_masks(n, seeds).view(np.int32))
    p1 = torch.empty((steps, nseq), dtype=torch.int32, device=dev())
    s1 = torch.empty((steps, nseq), dtype=torch.float32, device=dev())
    for t in range(steps):
        vs.vs_diversity_step_ref(Cd, Q1, m1, idx_out=p1[t], score_out=s1[t])
        vs.vs_diversity_accumulate(Cd, p1[t], Q1)
    m2 = T(seed_masks(n, seeds).view(np.int32))
    Q2 = torch.full((nseq, d), 3.0, dtype=torch.float32, device=dev())  # overwritten by the call
    p2, s2, Q2 = vs.vs_diversity_run_ref(Cd, T(seeds), m2, steps, Q=Q2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(m1, m2)
    assert torch.equal(Q1.view(torch.int32), Q2.view(torch.int32))
