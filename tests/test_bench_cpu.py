"""The bench's oracle leg on the CPU (no GPU): its parity verdict passes the
oracle's own answer and fails a planted error, its checked sets are the ones
the bench line names, and the line's single-GPU contract holds.

The GPU output is stood in for by the oracle's answer rounded to fp32 (an
object with the .cpu().numpy() of a tensor), so this checks the leg's
plumbing -- which rows it checks, how it calls the acceptance rule, what it
reports -- not the kernels.
"""
import os
import subprocess
import sys

import numpy as np

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Host:
    """Stands in for a device tensor: .cpu().numpy() gives the array."""

    def __init__(self, a):
        self.a = a

    def cpu(self):
        return self

    def numpy(self):
        return self.a


def _dense_outputs(w, idx=None):
    o_idx, o_val, _ = oracle.dense(w["Q"], w["C"], 0, threads=8)
    idx = o_idx if idx is None else idx
    return dict(idx=_Host(idx.astype(np.int32)), score=_Host(o_val.astype(np.float32)))


def test_dense_leg_checks_every_query_and_passes():
    w = synth.workload(1)
    w["gpu_out"] = _dense_outputs(w)
    base, parity = bench.cpu_baseline(1, w, 1.0)
    assert parity["pass"] and parity["checked"] == 256 and parity["same_index"] == 256
    assert parity["set"] == "all 256 queries"
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0
    assert base["one_thread_value"] > 0 and base["cpu_model"]


def test_dense_leg_fails_a_wrong_index():
    w = synth.workload(1)
    o_idx, _, o_gap = oracle.dense(w["Q"], w["C"], 0, threads=8)
    bad = o_idx.copy()
    r = int(np.argmax(o_gap))
    bad[r] = (bad[r] + 1) % w["nc"]
    w["gpu_out"] = _dense_outputs(w, bad)
    _, parity = bench.cpu_baseline(1, w, 1.0)
    assert not parity["pass"] and parity["same_index"] == 255
    assert any("outside the gap" in f for f in parity["failures"])


def test_dense_leg_uses_the_seeded_subset():
    """The 512x512-map workload is checked on its seeded 1,024-query subset:
    a wrong index on a query outside the subset is not seen, one inside is."""
    w = synth.workload(1)
    sel = synth.sample_queries(w["nq"], 64, key=1)
    w["subset"] = sel
    o_idx, _, _ = oracle.dense(w["Q"], w["C"], 0, threads=8)
    outside = int(np.setdiff1d(np.arange(w["nq"]), sel)[0])
    bad = o_idx.copy()
    bad[outside] = (bad[outside] + 1) % w["nc"]
    w["gpu_out"] = _dense_outputs(w, bad)
    _, parity = bench.cpu_baseline(1, w, 1.0)
    assert parity["pass"] and parity["checked"] == 64
    bad[sel[5]] = (bad[sel[5]] + 1) % w["nc"]
    w["gpu_out"] = _dense_outputs(w, bad)
    _, parity = bench.cpu_baseline(1, w, 1.0)
    assert not parity["pass"]


def test_diversity_replay_leg():
    """The diversity leg replays every pick against the Gram matrix and
    checks the final masks (16 sequences of the 8,359 x 768 table, 8 steps);
    a final mask with one bit more or less fails it."""
    from parity import check
    w = synth.workload(3)
    seeds = w["seeds"][:16]
    picks, vals = oracle.div_run(w["C"], seeds, 8)
    n = w["n"]
    W = (n + 31) // 32
    masks = np.zeros((16, W), np.uint32)
    for s in range(16):
        for p in [seeds[s], *picks[s]]:
            masks[s, p // 32] |= np.uint32(1 << (p % 32))
    w.update(seeds=seeds, nseq=16, reference="last", steps=8)
    w["gpu_out"] = dict(picks=_Host(picks.T.copy()), scores=_Host(vals.T.astype(np.float32).copy()),
                        mask=_Host(masks.view(np.int32)), steps=8)
    par = bench._div_parity(w, 8, check)
    assert par["pass"] and par["checked"] == 128
    bad_masks = masks.copy()
    bad_masks[3, 0] ^= np.uint32(1 << 30)  # one bit more or less than seed + picks
    w["gpu_out"]["mask"] = _Host(bad_masks.view(np.int32))
    assert not bench._div_parity(w, 8, check)["pass"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_replicates_off_under_a_profiler(monkeypatch):
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.under_profiler()
    monkeypatch.delenv("LD_PRELOAD")
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    assert not bench.under_profiler()


def test_traffic_hash_follows_code_not_comments():
    """A recorded traffic figure stays valid across comment edits and is
    dropped when the kernel's code changes."""
    code = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only(
        "/* header\n   text */\nint f(int x) {\n    // note\n    return x + 1;\n}\n\n")
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))
    for k in bench.KERNEL_SOURCES:
        assert len(bench.kernel_source_hash(k)) == 16
