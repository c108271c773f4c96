#!/usr/bin/env python3
"""Benchmark: query x candidate distance pairs per second on one MI355X.

Default workload: the dense best-matching-unit search of a 512x512 SOM map --
65,536 queries x 262,144 neurons, both N(0,1), d = 256, squared-L2 argmin --
with inputs resident in HBM.  One step = one vs_bmu_search call: candidate
(and query) norms, the fused MFMA scan with its arg-reduction and merge, and
the finalize kernel.

Output: one JSON line with the throughput (whole timed region), the per-step
median / min / max from HIP events between the steps, the spread over
independent process replicates, the roofline of the dominant kernel (its
algorithmic FLOPs per launch over its average launch time, taken with HIP
events on the launch stream by the library's timing hook), a CPU baseline --
the fp64 oracle timed on the workload's checked set on the host's cores, plus
a one-thread rate -- and the parity verdict of the timed run's own output
against that oracle run (the acceptance rule of tests/parity.py).  The small
32x32-map workload adds its per-call latency against an empty-kernel floor on
the same stream, eager and as a captured HIP graph.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]
                    [--replicates R] [--no-cpu-baseline] [--traffic-json FILE]
                    [--som [--som-sigma S --som-radius R]]

--som turns a BMU workload (1, 2, 4, 5) into SOM training: one step = one
epoch (vs_som_epoch / vs_som_epoch_csr: search, quantisation error, batch
update of the codebook in place) on the workload's map; the line adds the
epoch's per-phase times.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query×candidate distance pairs/sec (BMU search) + % of fp32 MFMA/HBM roof"
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# L2 -> CU read bandwidth of the whole chip in the sparse kernel's own access
# shape (four 256-byte row segments per 16-byte-per-lane load, a 4 MiB slice
# per XCD), measured with `bench.py --roof l2` (kernel in csrc/roofs.hip);
# the sparse scan is served from L2, so this is its roof
PEAK_L2_WIDE_GBS = 28795.7  # the highest of the runs on four machines (28,072 to 28,795.7)
# Row-gather rate of the diversity run from the Gram matrix: the run's own
# reference rows read whole, in the run's order, with nothing else in the
# loop (`bench.py --roof gather`, kernel in csrc/roofs.hip).  The 280 MB Gram
# matrix is served partly by the 256 MB last-level cache, so this exceeds
# the 8 TB/s HBM peak; it is the roof of the last-pick Gram run.
PEAK_GRAM_GATHER_GBS = 8694.5  # the highest of the runs on three machines (8,402.7 to 8,694.5)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (and with it the parity verdict)")
    ap.add_argument("--replicates", type=int, default=3,
                    help="independent processes timing the same steps (this one included); "
                         "their spread is reported.  Runs under a profiler use 1")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--dense-mode", choices=["fused", "unfused"], default="fused",
                    help="dense workloads: 'unfused' writes the whole score block, then "
                         "ranks each row in a second pass (the fusion comparator)")
    ap.add_argument("--div-mode", choices=["step", "gram"], default="step",
                    help="diversity workload: 'step' runs the MFMA scan every step, 'gram' "
                         "builds the table's Gram matrix once per run and scans one row of it "
                         "per sequence and step")
    ap.add_argument("--div-ref", choices=["last", "centroid"], default="last",
                    help="diversity reference: the last pick, or the centroid of the "
                         "sequence so far (per-step scan against explicit reference rows)")
    ap.add_argument("--div-steps", default=None,
                    help="diversity steps per run: a number, or 'full' (every row of the "
                         "table, n - 1 picks); default the workload's 64")
    ap.add_argument("--csr-storage", choices=["f32", "f16"], default="f32",
                    help="sparse workload: codebook storage type ('f16': the 128-neuron "
                         "blocked fp16 copy, fp32 arithmetic)")
    ap.add_argument("--csr-layout", choices=["blocked", "plain"], default="blocked",
                    help="sparse workload: 'blocked' times the 64-neuron blocked copy of the "
                         "codebook plus the search over it, 'plain' the search over the "
                         "row-padded feature-major codebook")
    ap.add_argument("--som", action="store_true",
                    help="one step = one SOM epoch around the search (workloads 1, 2, 4, 5)")
    ap.add_argument("--som-sigma", type=float, default=2.0,
                    help="Gaussian neighbourhood width in map cells")
    ap.add_argument("--som-radius", type=int, default=6,
                    help="square window radius in map cells (default 3 sigma)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration mode: time a plain device copy of this many bytes "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--roof", choices=["l2", "mfma", "gather"], default=None,
                    help="measure a roof and exit: l2 = the on-chip read rate of the sparse "
                         "scan's access pattern (256-byte row loads from an L2-resident region "
                         "per XCD); mfma = the fp32 MFMA rate of a loop with no memory "
                         "traffic; gather = the rate of reading the diversity run's Gram rows "
                         "whole, in the run's order")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB",
                                                          "COPY_WRITE_DB"),
                    help="record HBM traffic per launch of the workload's dominant kernel from "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE databases of the workload and "
                         "of the --copy-bytes calibration run, then exit")
    ap.add_argument("--traffic-copy-bytes", type=int, default=268435456,
                    help="bytes read (and written) per launch of the calibration copy")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def load_traffic(path, kernel, workload):
    try:
        with open(path) as f:
            t = json.load(f)
        e = t.get(f"{workload}:{kernel}")
        if e and e.get("kernel_source_hash") == kernel_source_hash(kernel):
            return e.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


KERNEL_SOURCES = {"k_bmu_qreg": "bmu_qreg.hip", "k_bmu_q16": "bmu_q16.hip",
                  "k_small_scan": "bmu_small.hip",
                  "k_bmu_mfma": "bmu_mfma.hip", "k_bmu_csr": "bmu_csr.hip"}


def _code_only(text):
    """Source text without comments, trailing blanks or empty lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash(kernel):
    """Hash of the code (comments left out) of the kernel's source file and
    the shared header: a recorded traffic figure is reported only while
    both are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "farthest_vector_search_amd", "csrc")
    for name in (KERNEL_SOURCES[kernel], "vs_internal.h"):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ workloads --

def setup(k, torch, vs, a):
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    w = synth.workload(k)
    if w["kind"] == "dense":
        Q = torch.from_numpy(w["Q"]).to(dev)
        C = torch.from_numpy(w["C"]).to(dev)
        idx = torch.empty(w["nq"], dtype=torch.int32, device=dev)
        score = torch.empty(w["nq"], dtype=torch.float32, device=dev)
        ws = torch.empty(vs.lib().vs_bmu_search_workspace(w["nq"], w["nc"], w["d"], 0),
                         dtype=torch.uint8, device=dev)

        if a.dense_mode == "unfused":
            S = torch.empty((w["nq"], (w["nc"] + 63) // 64 * 64), dtype=torch.float32,
                            device=dev)

            def step():
                vs.vs_bmu_search_unfused(Q, C, 0, S=S, idx_out=idx, score_out=score,
                                         workspace=ws)
        else:
            def step():
                vs.vs_bmu_search(Q, C, 0, idx_out=idx, score_out=score, workspace=ws)
        w["gpu_out"] = dict(idx=idx, score=score)
        pairs = w["nq"] * w["nc"]
        flops = 2.0 * w["d"] * pairs
        cfg = dict(workload=w["name"], nq=w["nq"], nc=w["nc"], d=w["d"], metric="l2sq_min")
        if a.dense_mode == "unfused":
            cfg["mode"] = "unfused"
        return w, step, pairs, flops, 1, cfg
    if w["kind"] == "diversity":
        n, d, nseq, steps = w["n"], w["d"], w["nseq"], w["steps"]
        if a.div_steps is not None:
            steps = n - 1 if a.div_steps == "full" else int(a.div_steps)
        C = torch.from_numpy(w["C"]).to(dev)
        seeds = torch.from_numpy(w["seeds"]).to(dev)
        W = (n + 31) // 32
        m0 = np.zeros((nseq, W), np.uint32)
        m0[np.arange(nseq), w["seeds"] // 32] |= (np.uint32(1) << (w["seeds"] % 32).astype(np.uint32))
        mask0 = torch.from_numpy(m0.view(np.int32)).to(dev)
        mask = mask0.clone()
        picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev)
        # the timed runs write every pick's score too (one 4-byte store per
        # sequence and step), so the timed output is the one the oracle checks
        scores = torch.empty((steps, nseq), dtype=torch.float32, device=dev)
        w["gpu_out"] = dict(picks=picks, scores=scores, mask=mask, steps=steps)
        ws = torch.empty(vs.lib().vs_diversity_step_workspace(n, d, nseq), dtype=torch.uint8,
                         device=dev)

        if a.div_mode == "gram":
            # one run = the Gram matrix of the table (once) + `steps` scans of
            # one Gram row per sequence
            ldg = (n + 63) // 64 * 64
            Gbuf = torch.empty((n, ldg), dtype=torch.float32, device=dev)
            # algorithmic bytes of one run: the live (unmasked) entries of one
            # Gram row per sequence and step -- n - 1 - t at step t -- (with
            # the centroid reference also the running sums read and written),
            # the mask row read and written once, the seed read and one pick
            # written per step
            live = sum(max(n - 1 - t, 0) for t in range(steps)) / steps
            if a.div_ref == "centroid":
                Rbuf = torch.empty((nseq, ldg), dtype=torch.float32, device=dev)

                def step():
                    mask.copy_(mask0)
                    G = vs.vs_diversity_gram(C, out=Gbuf)
                    vs.vs_diversity_run_gram(G, seeds, mask, steps, R=Rbuf[:, :n],
                                             picks_out=picks, scores_out=scores)
                per_col = 12
            else:
                def step():
                    mask.copy_(mask0)
                    G = vs.vs_diversity_gram(C, out=Gbuf)
                    vs.vs_diversity_run_gram(G, seeds, mask, steps, picks_out=picks,
                                             scores_out=scores)
                per_col = 4
            w["run_bytes"] = nseq * (steps * (per_col * live + 4) + 8 * W + 4)
        elif a.div_ref == "centroid":
            # the reference of each sequence is the running sum of its rows
            # (the centroid times a positive count): start at the seed's row
            Q = torch.empty((nseq, d), dtype=torch.float32, device=dev)

            def step():
                mask.copy_(mask0)
                vs.vs_diversity_run_ref(C, seeds, mask, steps, Q=Q, picks_out=picks,
                                        scores_out=scores, workspace=ws)
        else:
            def step():
                mask.copy_(mask0)
                vs.vs_diversity_run(C, seeds, mask, steps, picks_out=picks, scores_out=scores,
                                    workspace=ws)
        pairs = nseq * n * steps
        flops = 2.0 * d * pairs
        w["reference"] = a.div_ref
        cfg = dict(workload=w["name"], n=n, d=d, nseq=nseq, steps_per_run=steps,
                   metric="cos_min_masked", mode=a.div_mode, reference=a.div_ref)
        return w, step, pairs, flops, steps, cfg
    # sparse
    indptr = torch.from_numpy(w["indptr"]).to(dev)
    indices = torch.from_numpy(w["indices"]).to(dev)
    values = torch.from_numpy(w["values"]).to(dev)
    # feature-major codebook with rows padded by 64 neurons: a row stride of
    # 65,536 floats (a power of two) would alias every row's slice onto the
    # same L2 sets
    nq, nc = w["nq"], w["nc"]
    CT = torch.empty((w["d"], nc + 64), dtype=torch.float32, device=dev)[:, :nc]
    CT.copy_(torch.from_numpy(w["CT"]).to(dev))
    idx = torch.empty(nq, dtype=torch.int32, device=dev)
    score = torch.empty(nq, dtype=torch.float32, device=dev)
    ws = torch.empty(vs.lib().vs_bmu_search_csr_workspace(nq, nc, w["d"], 0), dtype=torch.uint8,
                     device=dev)

    if a.csr_storage == "f16":
        # each step writes the fp16 blocked copy of the fp32 codebook and
        # searches it (load fp16, compute fp32)
        CB16 = torch.empty(vs.lib().vs_csr_blocked_f16_bytes(nc, w["d"]) // 2,
                           dtype=torch.float16, device=dev)

        def step():
            vs.vs_csr_block_codebook_f16(CT, out=CB16)
            vs.vs_bmu_search_csr_blocked_f16(indptr, indices, values, CB16, nc, 0, d=w["d"],
                                             idx_out=idx, score_out=score, workspace=ws)
    elif a.csr_layout == "plain":
        def step():
            vs.vs_bmu_search_csr(indptr, indices, values, CT, 0, idx_out=idx, score_out=score,
                                 workspace=ws)
    else:
        # each step re-blocks the feature-major codebook (as a caller holding
        # it feature-major would) and searches the blocked copy
        CB = torch.empty(vs.lib().vs_csr_blocked_bytes(nc, w["d"]) // 4, dtype=torch.float32,
                         device=dev)

        def step():
            vs.vs_csr_block_codebook(CT, out=CB)
            vs.vs_bmu_search_csr_blocked(indptr, indices, values, CB, nc, 0, d=w["d"],
                                         idx_out=idx, score_out=score, workspace=ws)
    w["gpu_out"] = dict(idx=idx, score=score)
    pairs = nq * nc
    w["nnz"] = int(w["indices"].shape[0])
    flops = 2.0 * w["nnz"] * nc
    cfg = dict(workload=w["name"], nq=nq, nc=nc, d=w["d"], nnz=w["nnz"], metric="l2sq_min",
               codebook_row_stride=nc + 64,
               codebook_layout="blocked" if a.csr_storage == "f16" else a.csr_layout,
               codebook_storage=a.csr_storage)
    w["value_bytes"] = 2 if a.csr_storage == "f16" else 4
    chunks = (nc + (127 if a.csr_storage == "f16" else 63)) // (128 if a.csr_storage == "f16" else 64)
    rounds = (chunks + min(8, chunks) - 1) // min(8, chunks)  # one scan launch per round
    return w, step, pairs, flops, rounds, cfg


SOM_MAPS = {1: (32, 32), 2: (128, 128), 4: (256, 256), 5: (512, 512)}


def setup_som(k, torch, vs, a):
    """One step = one SOM epoch on workload k's inputs and codebook (the map
    trains on from step to step, as successive epochs do)."""
    import synth
    if k not in SOM_MAPS:
        raise SystemExit(f"--som needs a BMU workload ({sorted(SOM_MAPS)})")
    dev = torch.device("cuda:0")
    w = synth.workload(k)
    rows, cols = SOM_MAPS[k]
    sig, R = a.som_sigma, a.som_radius
    nq, nc, d = w["nq"], w["nc"], w["d"]
    L = vs.lib()
    bmu = torch.empty(nq, dtype=torch.int32, device=dev)
    score = torch.empty(nq, dtype=torch.float32, device=dev)
    qe = torch.empty(1, dtype=torch.float64, device=dev)
    phases = {}
    if w["kind"] == "dense":
        X = torch.from_numpy(w["Q"]).to(dev)
        C = torch.from_numpy(w["C"]).to(dev)
        ws = torch.empty(L.vs_som_epoch_workspace(nq, rows, cols, d), dtype=torch.uint8,
                         device=dev)
        ws_s = torch.empty(L.vs_bmu_search_workspace(nq, nc, d, 0), dtype=torch.uint8, device=dev)
        ws_u = torch.empty(L.vs_som_update_workspace(rows, cols, d), dtype=torch.uint8,
                           device=dev)

        def step():
            vs.vs_som_epoch(X, C, (rows, cols), sig, R, bmu_out=bmu, score_out=score, qe_out=qe,
                            workspace=ws)
        phases["search"] = lambda: vs.vs_bmu_search(X, C, 0, idx_out=bmu, score_out=score,
                                                    workspace=ws_s)
        phases["update"] = lambda: vs.vs_som_update(X, bmu, C, (rows, cols), sig, R,
                                                    workspace=ws_u)
        in_bytes = nq * d * 4
        flops = 2.0 * d * nq * nc
        launches = 1
    else:
        indptr = torch.from_numpy(w["indptr"]).to(dev)
        indices = torch.from_numpy(w["indices"]).to(dev)
        values = torch.from_numpy(w["values"]).to(dev)
        CB = vs.vs_csr_block_codebook(torch.from_numpy(w["CT"]).to(dev))
        torch.cuda.synchronize()
        ws = torch.empty(L.vs_som_epoch_csr_workspace(nq, rows, cols, d), dtype=torch.uint8,
                         device=dev)
        ws_s = torch.empty(L.vs_bmu_search_csr_workspace(nq, nc, d, 0), dtype=torch.uint8,
                           device=dev)
        ws_u = torch.empty(L.vs_som_update_workspace(rows, cols, d), dtype=torch.uint8,
                           device=dev)

        if a.csr_storage == "f16":
            # the search runs over an fp16 copy remade from the fp32 codebook
            # each epoch; the update keeps the fp32 weights
            CB16 = torch.empty(L.vs_csr_blocked_f16_bytes(nc, d) // 2, dtype=torch.float16,
                               device=dev)

            def step():
                vs.vs_som_epoch_csr_f16(indptr, indices, values, CB, (rows, cols), d, sig, R,
                                        CB16=CB16, bmu_out=bmu, score_out=score, qe_out=qe,
                                        workspace=ws)

            def search_phase():
                vs.vs_csr_blocked_to_f16(CB, nc, d, out=CB16)
                vs.vs_bmu_search_csr_blocked_f16(indptr, indices, values, CB16, nc, 0, d=d,
                                                 idx_out=bmu, score_out=score, workspace=ws_s)
            phases["search"] = search_phase
        else:
            def step():
                vs.vs_som_epoch_csr(indptr, indices, values, CB, (rows, cols), d, sig, R,
                                    bmu_out=bmu, score_out=score, qe_out=qe, workspace=ws)
            phases["search"] = lambda: vs.vs_bmu_search_csr_blocked(
                indptr, indices, values, CB, nc, 0, d=d, idx_out=bmu, score_out=score,
                workspace=ws_s)
        phases["update"] = lambda: vs.vs_som_update_csr(indptr, indices, values, bmu, CB,
                                                        (rows, cols), d, sig, R, workspace=ws_u)
        w["nnz"] = int(w["indices"].shape[0])
        f16 = a.csr_storage == "f16"
        w["value_bytes"] = 2 if f16 else 4
        in_bytes = w["nnz"] * 8 + (nq + 1) * 4
        flops = 2.0 * w["nnz"] * nc
        chunks = (nc + (127 if f16 else 63)) // (128 if f16 else 64)
        launches = (chunks + min(8, chunks) - 1) // min(8, chunks)
    phases["qe"] = lambda: vs.vs_som_qe(score, qe_out=qe)
    # the update's algorithmic HBM bytes: read the inputs and their BMUs once,
    # write every neuron's new weights once
    w["update_bytes"] = in_bytes + nq * 4 + nc * d * 4
    w["som_phases"] = phases
    w["som_qe"] = qe
    cfg = dict(workload=w["name"] + "+som_epoch", nq=nq, nc=nc, d=d, map=f"{rows}x{cols}",
               sigma=sig, radius=R, metric="l2sq_min",
               update="batch map, Gaussian in a square window, separable passes")
    if w["kind"] == "csr":
        cfg.update(nnz=w["nnz"], codebook_layout="blocked", codebook_storage=a.csr_storage)
    return w, step, nq * nc, flops, launches, cfg


def som_phase_times(w, torch, reps=3):
    """Mean ms of each phase of the epoch, run as the separate entry points
    the epoch calls, bracketed by events on the current stream."""
    out = {}
    for name in ("search", "qe", "update"):
        fn = w["som_phases"][name]
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
    ub = w["update_bytes"]
    out["update_algorithmic_bytes"] = ub
    out["update_GBps"] = round(ub / (out["update_ms"] * 1e-3) / 1e9, 1)
    out["update_frac_hbm"] = round(out["update_GBps"] / PEAK_HBM_GBS, 4)
    return out


def cpu_baseline_som(k, w, target_s):
    """Oracle epoch on a bounded sample: the exact search on a sample of
    inputs plus the update of a sample of neurons (BMUs drawn uniformly),
    scaled to the whole epoch."""
    import numpy as np
    import oracle
    import synth
    threads = oracle.default_threads()
    rows, cols = SOM_MAPS[k]
    nq, nc, d = w["nq"], w["nc"], w["d"]
    half = target_s / 2
    if w["kind"] == "dense":
        t0 = time.perf_counter()
        oracle.dense(w["Q"][:threads], w["C"], 0, threads=threads)
        per_q = (time.perf_counter() - t0) / threads
        ns = int(max(threads, min(nq, half / max(per_q, 1e-9))))
        t0 = time.perf_counter()
        oracle.dense(w["Q"][:ns], w["C"], 0, threads=threads)
        search_s = (time.perf_counter() - t0) * nq / ns
        ip, ix, vv = oracle.dense_as_csr(w["Q"])
        C_old = w["C"]
        old = None
    else:
        col_sq = oracle.sqnorms(w["CT"], feature_major=True, threads=threads)
        ptr = w["indptr"]
        t0 = time.perf_counter()
        oracle.csr(ptr[:threads + 1], w["indices"], w["values"], w["CT"], 0, col_sq=col_sq,
                   threads=threads)
        per_q = (time.perf_counter() - t0) / threads
        ns = int(max(threads, min(nq, half / max(per_q, 1e-9))))
        t0 = time.perf_counter()
        oracle.csr(ptr[:ns + 1], w["indices"], w["values"], w["CT"], 0, col_sq=col_sq,
                   threads=threads)
        search_s = (time.perf_counter() - t0) * nq / ns
        ip, ix, vv = w["indptr"], w["indices"], w["values"]
        C_old = None
    bmu = synth.random_indices(nq, nc, key=k)
    probe = np.arange(threads, dtype=np.int32)
    kw = {} if C_old is not None else {"old_rows": np.ascontiguousarray(w["CT"][:, probe].T)}
    t0 = time.perf_counter()
    oracle.som_update(ip, ix, vv, d, bmu, C_old, rows, cols, 2.0, 6, neurons=probe,
                      threads=threads, **kw)
    per_n = (time.perf_counter() - t0) / threads
    nn = int(max(threads, min(nc, half / max(per_n, 1e-9))))
    sel = synth.sample_queries(nc, nn, key=k).astype(np.int32)
    kw = {} if C_old is not None else {"old_rows": np.ascontiguousarray(w["CT"][:, sel].T)}
    t0 = time.perf_counter()
    oracle.som_update(ip, ix, vv, d, bmu, C_old, rows, cols, 2.0, 6, neurons=sel,
                      threads=threads, **kw)
    dt_u = time.perf_counter() - t0
    update_s = dt_u * nc / nn
    epoch_s = search_s + update_s
    return dict(value=nq * nc / epoch_s, unit="pairs/s", cores=threads, kind="oracle",
                sample=(f"search of {ns} of {nq} inputs x all {nc} neurons and update of {nn} "
                        f"of {nc} neurons, scaled to one epoch"),
                epoch_s=round(epoch_s, 2), search_s=round(search_s, 2),
                update_s=round(update_s, 2))


# ------------------------------------------------------------ cpu leg --

def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _verdict(fails, stats, checked_set):
    out = {"checked": stats["rows"], "set": checked_set, "pass": not fails}
    out.update({k: stats[k] for k in ("same_index", "gap_accepted", "empty", "floor_bound")})
    if fails:
        out["failures"] = fails[:3]
    return out


def _one_thread_rate(run, unit_pairs, first=2, target_s=1.5):
    """Pairs/s of the single-threaded oracle: time `first` units, then enough
    units for about target_s seconds; run(m) scans m units."""
    t0 = time.perf_counter()
    run(first)
    per = (time.perf_counter() - t0) / first
    m = max(first, int(target_s / max(per, 1e-9)))
    t0 = time.perf_counter()
    m = run(m)
    dt = time.perf_counter() - t0
    return m * unit_pairs / dt, m


def cpu_baseline(k, w, target_s):
    """Oracle (fp64, plain loops, untuned) on the workload's checked set, all
    host threads, each running the single-threaded scan on its own shard;
    the result is also the parity verdict of the timed GPU output.  Returns
    (cpu_baseline dict, parity dict or None)."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import check, l2_floor
    threads = oracle.default_threads()
    base = dict(unit="pairs/s", cores=threads, kind="oracle", cpu_model=cpu_model())
    if w["kind"] == "dense":
        nc, nq = w["nc"], w["nq"]
        # checked set: every query, or the workload's seeded subset
        sel = w.get("subset")
        label = (f"the seeded {len(sel)}-query subset" if sel is not None
                 else f"all {nq} queries")
        sel = np.arange(nq) if sel is None else np.asarray(sel)
        Qs = np.ascontiguousarray(w["Q"][sel])
        base["one_thread_value"], m1 = _one_thread_rate(
            lambda m: (oracle.dense(Qs[:m], w["C"], 0, threads=1), min(m, len(sel)))[1], nc)
        t0 = time.perf_counter()
        o_idx, o_val, o_gap = oracle.dense(Qs, w["C"], 0, threads=threads)
        dt = time.perf_counter() - t0
        base.update(value=len(sel) * nc / dt, seconds=round(dt, 2),
                    sample=f"{label} x all {nc} candidates (the checked set)",
                    one_thread_sample=f"{m1} queries x all {nc} candidates, one thread")
        parity = None
        if "gpu_out" in w:
            idx = w["gpu_out"]["idx"].cpu().numpy()[sel]
            score = w["gpu_out"]["score"].cpu().numpy()[sel]
            fails, stats = check(idx, score, o_idx, o_val, o_gap, 0, l2_floor(Qs, w["C"], o_idx),
                                 lambda r, c: oracle.pair_values(Qs, w["C"], 0, r, c))
            parity = _verdict(fails, stats, label)
        return base, parity
    if w["kind"] == "diversity":
        n = w["n"]
        # the value: one step straight from the rows (no Gram cache) for a
        # sample of sequences, each scanning all n rows against its reference
        base["one_thread_value"], m1 = _one_thread_rate(
            lambda m: (oracle.div_run(w["C"], w["seeds"][:m], 1), m)[1], n)
        t0 = time.perf_counter()
        oracle.div_run(w["C"], w["seeds"][:2], 1)
        per_seq = (time.perf_counter() - t0) / 2
        nsample = int(max(threads, min(w["nseq"], target_s * threads / max(per_seq, 1e-9))))
        seeds = w["seeds"][:nsample]
        from concurrent.futures import ThreadPoolExecutor
        parts = np.array_split(seeds, threads)
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda s: oracle.div_run(w["C"], s, 1), [p for p in parts if len(p)]))
        dt = time.perf_counter() - t0
        base.update(value=nsample * n / dt, seconds=round(dt, 2),
                    sample=f"one step of {nsample} of {w['nseq']} sequences x all {n} rows",
                    one_thread_sample=f"one step of {m1} sequences x all {n} rows, one thread")
        return base, _div_parity(w, threads, check)
    # sparse: the 4,096 seeded rows
    ptr = w["indptr"]
    nc = w["nc"]
    sel = synth_sample(w["nq"], 4096, key=4)
    sub_ptr = np.concatenate([[0], np.cumsum(ptr[sel + 1] - ptr[sel])]).astype(np.int32)
    sub_idx = np.concatenate([w["indices"][ptr[i]:ptr[i + 1]] for i in sel])
    sub_val = np.concatenate([w["values"][ptr[i]:ptr[i + 1]] for i in sel])
    col_sq = oracle.sqnorms(w["CT"], feature_major=True, threads=threads)

    def rows(m):
        oracle.csr(sub_ptr[:m + 1], sub_idx, sub_val, w["CT"], 0, col_sq=col_sq, threads=1)
        return m
    base["one_thread_value"], m1 = _one_thread_rate(rows, nc)
    t0 = time.perf_counter()
    o_idx, o_val, o_gap = oracle.csr(sub_ptr, sub_idx, sub_val, w["CT"], 0, col_sq=col_sq,
                                     threads=threads)
    dt = time.perf_counter() - t0
    base.update(value=len(sel) * nc / dt, seconds=round(dt, 2),
                sample=f"the seeded {len(sel)} of {w['nq']} CSR rows x all {nc} neurons "
                       "(the checked set)",
                one_thread_sample=f"{m1} CSR rows x all {nc} neurons, one thread")
    parity = None
    if "gpu_out" in w and w.get("value_bytes", 4) == 4:
        idx = w["gpu_out"]["idx"].cpu().numpy()[sel]
        score = w["gpu_out"]["score"].cpu().numpy()[sel]
        qn = np.array([np.sum(sub_val[sub_ptr[i]:sub_ptr[i + 1]].astype(np.float64) ** 2)
                       for i in range(len(sel))])

        def pick_values(r, c):
            return np.array([oracle.csr(np.array([0, sub_ptr[i + 1] - sub_ptr[i]], np.int32),
                                        sub_idx[sub_ptr[i]:sub_ptr[i + 1]],
                                        sub_val[sub_ptr[i]:sub_ptr[i + 1]],
                                        np.ascontiguousarray(w["CT"][:, j:j + 1]), 0,
                                        col_sq=col_sq[j:j + 1])[1][0] for i, j in zip(r, c)])
        fails, stats = check(idx, score, o_idx, o_val, o_gap, 0, 1e-2 * (qn + 1.0), pick_values)
        parity = _verdict(fails, stats, f"the seeded {len(sel)} CSR rows")
    return base, parity


def synth_sample(nq, count, key):
    import synth
    return synth.sample_queries(nq, count, key=key)


def _div_parity(w, threads, check):
    """Replay of every pick of the timed run (last-pick reading, at most the
    workload's 64 steps) against the oracle's fp64 cosine Gram matrix, plus
    the final masks = seed + picks."""
    import numpy as np
    import oracle
    g = w.get("gpu_out")
    if g is None or w.get("reference", "last") != "last" or g["steps"] > w["steps"]:
        return None
    picks = g["picks"].cpu().numpy().T.copy()      # [nseq, steps]
    scores = g["scores"].cpu().numpy().T.copy()
    masks = g["mask"].cpu().numpy().view(np.uint32)
    n, seeds = w["n"], w["seeds"]
    G = oracle.gram_cos(w["C"], threads=threads)
    rep = oracle.div_replay(G, seeds, picks, threads=threads)
    del G
    live = rep["bidx"] >= 0
    fails = []
    if not (rep["pick_ok"][live] == 1).all():
        fails.append("illegal pick (masked or out of range)")
    if not (picks[~live] == -1).all():
        fails.append("pick where nothing was left")
    flat = lambda a: a.reshape(-1)  # noqa: E731
    f, stats = check(flat(picks), flat(scores), flat(rep["bidx"]), flat(rep["best"]),
                     flat(rep["gap"]), 3, 1e-2, lambda r, c: flat(rep["pick_value"])[r],
                     legal=lambda r, c: flat(rep["pick_ok"])[r] == 1)
    fails += f
    exp = np.zeros_like(masks)
    rows = np.arange(len(seeds))
    exp[rows, seeds // 32] |= (np.uint32(1) << (seeds % 32).astype(np.uint32))
    for t in range(picks.shape[1]):
        p = picks[:, t]
        ok = p >= 0
        np.bitwise_or.at(exp, (rows[ok], p[ok] // 32), np.uint32(1) << (p[ok] % 32).astype(np.uint32))
    if not np.array_equal(exp, masks):
        fails.append("final masks differ from seed + picks")
    return _verdict(fails, stats, f"every pick of {len(seeds)} sequences x {picks.shape[1]} steps")


def _pmc_avg(db, counter, name_prefix):
    """Average per-dispatch value (KiB) of a counter for kernels whose name
    starts with name_prefix (after 'void ' and the namespace)."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, value from counters_collection where counter_name = ?",
                     (counter,)).fetchall()
    vals = [v for k, v in rows if k.replace("void ", "").replace("vs::", "").startswith(name_prefix)]
    if not vals:
        raise SystemExit(f"{db}: no {counter} samples for {name_prefix}")
    return sum(vals) / len(vals), len(vals)


DOMINANT = {1: "k_small_scan", 2: "k_bmu_qreg", 3: "k_bmu_q16", 4: "k_bmu_csr", 5: "k_bmu_qreg"}


def record_traffic(a):
    """FETCH_SIZE and WRITE_SIZE count KiB per dispatch; each is scaled by
    what the same counter reads for a plain copy of known size."""
    import synth
    f_db, w_db, cf_db, cw_db = a.traffic_from
    kernel = DOMINANT[a.workload]
    copy_kib = a.traffic_copy_bytes / 1024.0
    cf, _ = _pmc_avg(cf_db, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    cw, _ = _pmc_avg(cw_db, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    f, nf = _pmc_avg(f_db, "FETCH_SIZE", kernel)
    w, nw = _pmc_avg(w_db, "WRITE_SIZE", kernel)
    fs, ws = copy_kib / cf, copy_kib / cw
    total = (f * fs + w * ws) * 1024.0
    name = synth.WORKLOADS[a.workload]["name"]
    try:
        with open(a.traffic_json) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[f"{name}:{kernel}"] = {
        "bytes_per_launch": round(total), "fetch_kib_raw": round(f, 1),
        "write_kib_raw": round(w, 1), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "dispatches": [nf, nw], "kernel_source_hash": kernel_source_hash(kernel)}
    with open(a.traffic_json, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    print(json.dumps({name: table[f"{name}:{kernel}"]}))


def measure_l2_roof(a, torch):
    """L2 -> CU read bandwidth for row segments read the way the sparse scan
    reads the codebook: each XCD reads its own 4 MiB region, 16 loads in
    flight per wave, 16 waves per CU, in three shapes:
    one 256-byte row per 4-byte-per-lane load, four 256-byte rows per
    16-byte-per-lane load (the shape of the sparse kernel), and one 1 KiB row
    per 16-byte-per-lane load."""
    import ctypes
    from farthest_vector_search_amd.build import ROOF_LIB
    L = ctypes.CDLL(ROOF_LIB)
    L.vs_roof_l2_read.restype = ctypes.c_int64
    L.vs_roof_l2_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    wg_per_xcd = n_cu // 8 * 4
    out = torch.empty(8 * wg_per_xcd * 4, device="cuda:0")
    res = {}
    # 4 MiB per XCD in every shape, the size of one 64-neuron slice of the
    # 16,384-feature codebook in the blocked layout (256-byte rows, no gaps)
    shapes = (("dword_256B", 1, 1, 16384, 64), ("dwordx4_4x256B", 4, 4, 16384, 64),
              ("dwordx4_1KiB", 4, 1, 4096, 256))
    for name, vw, rpi, rows, ld in shapes:
        buf = torch.rand(8 * rows * ld, device="cuda:0")
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        passes = 64
        args = (ctypes.c_void_p(buf.data_ptr()), rows, ld, passes, vw, rpi, wg_per_xcd,
                ctypes.c_void_p(out.data_ptr()), stream)
        L.vs_roof_l2_read(*args)  # warm the L2s
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nbytes = 0
        for _ in range(a.steps):
            nbytes += L.vs_roof_l2_read(*args)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        res[name] = dict(GBps=round(nbytes / ms / 1e6, 1), bytes_per_launch=nbytes // a.steps,
                         ms_per_launch=round(ms / a.steps, 4),
                         region_bytes_per_xcd=rows * ld * 4)
        del buf
    print(json.dumps({"l2_roof": res}), flush=True)


def measure_mfma_roof(a, torch):
    """The fp32 MFMA rate this part sustains with no memory traffic: every
    wave issues MFMAs over two independent accumulator chains (the
    dependence pattern of the dense scans), one workgroup per CU, for 1, 2
    and 4 waves per SIMD; 32x32x2 and 16x16x4 shapes.  Against the
    published 157.3 TFLOP/s this is the highest fraction a dense scan can
    reach here."""
    import ctypes
    from farthest_vector_search_amd.build import ROOF_LIB
    L = ctypes.CDLL(ROOF_LIB)
    L.vs_roof_mfma.restype = ctypes.c_int64
    L.vs_roof_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(n_cu * 256 * 4, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for shape in (32, 16):
        for wps in (1, 2, 4):
            iters = 4000 if shape == 32 else 8000
            args = (shape, wps, iters, n_cu, ctypes.c_void_p(out.data_ptr()), stream)
            if L.vs_roof_mfma(*args) < 0:
                raise RuntimeError("vs_roof_mfma rejected its arguments")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            flop = 0
            for _ in range(a.steps):
                flop += L.vs_roof_mfma(*args)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            tf = flop / ms / 1e9
            res[f"{shape}x{shape}_waves_per_simd_{wps}"] = dict(
                TFLOPs=round(tf, 2), frac_of_published=round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                ms_per_launch=round(ms / a.steps, 4), flop_per_launch=flop // a.steps)
    print(json.dumps({"mfma_roof": res}), flush=True)


def measure_gather_roof(a, torch):
    """Row-gather rate of the diversity run from the Gram matrix.  The 8,359
    x 768 table's Gram matrix (8,359 x 8,384 fp32, 280 MB: more than the
    256 MB last-level cache) is built, one 64-step run of the 3,584
    sequences gives the run's own reference rows (the seed, then the picks of
    steps 0 .. 62), and k_gather_roof reads those rows whole, in the run's
    order, with nothing else in the loop; for comparison the same number of
    uniformly random rows."""
    import ctypes
    import numpy as np
    import synth
    import farthest_vector_search_amd as vs
    from farthest_vector_search_amd.build import ROOF_LIB
    L = ctypes.CDLL(ROOF_LIB)
    L.vs_roof_gather.restype = ctypes.c_int32
    L.vs_roof_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    w = synth.workload(3)
    n, nseq, steps = w["n"], w["nseq"], w["steps"]
    C = torch.from_numpy(w["C"]).to(dev)
    seeds = torch.from_numpy(w["seeds"]).to(dev)
    W = (n + 31) // 32
    m0 = np.zeros((nseq, W), np.uint32)
    m0[np.arange(nseq), w["seeds"] // 32] |= (np.uint32(1) << (w["seeds"] % 32).astype(np.uint32))
    mask = torch.from_numpy(m0.view(np.int32)).to(dev)
    ldg = (n + 63) // 64 * 64
    G = vs.vs_diversity_gram(C, out=torch.empty((n, ldg), dtype=torch.float32, device=dev))
    picks = torch.empty((steps, nseq), dtype=torch.int32, device=dev)
    vs.vs_diversity_run_gram(G, seeds, mask, steps, picks_out=picks, want_scores=False)
    run_rows = torch.cat([seeds[None], picks[:-1]]).contiguous()
    (r,) = synth.rng_children(77, 1)
    rand_rows = torch.from_numpy(r.integers(0, n, (steps, nseq), dtype=np.int32)).to(dev)
    grid = nseq
    out = torch.empty(grid * 256, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, rows in (("run_rows", run_rows), ("random_rows", rand_rows)):
        valid = int(((rows >= 0) & (rows < n)).sum())
        args = (ctypes.c_void_p(G.data_ptr()), n, n, ldg, ctypes.c_void_p(rows.data_ptr()), nseq,
                steps, grid, ctypes.c_void_p(out.data_ptr()), stream)
        if L.vs_roof_gather(*args) != 0:
            raise RuntimeError("vs_roof_gather rejected its arguments")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            L.vs_roof_gather(*args)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        nbytes = valid * n * 4
        res[name] = dict(GBps=round(nbytes / ms / 1e6, 1), bytes_per_launch=nbytes,
                         ms_per_launch=round(ms, 4), table_bytes=n * ldg * 4)
    print(json.dumps({"gather_roof": res}), flush=True)


def copy_calibration(a, torch):
    """A plain copy of known size (read n bytes, write n bytes) per launch."""
    n = a.copy_bytes // 4
    src = torch.rand(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(a.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(a.steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                      "launches": a.steps + a.warmup, "ms_per_copy": ms,
                      "GBps_read_plus_write": 2 * n * 4 / ms / 1e6}), flush=True)


def under_profiler():
    """True inside rocprofv3 (its tool library is preloaded and its settings
    are in the environment): no child processes are started there."""
    return ("rocprof" in os.environ.get("LD_PRELOAD", "")
            or any(k.startswith("ROCPROF") for k in os.environ))


def run_replicates(a, count):
    """count - 1 further processes run the same timed steps (no oracle leg),
    one after the other, before this process touches the GPU; returns their
    JSON lines."""
    import subprocess
    argv = [x for x in sys.argv[1:]]
    out = []
    for r in range(count - 1):
        cmd = [sys.executable, os.path.abspath(__file__), *argv, "--replicates", "1",
               "--no-cpu-baseline", "--child"]
        log(f"replicate process {r + 1} of {count - 1}")
        p = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        if p.returncode != 0:
            sys.stderr.write(p.stderr[-2000:])
            raise SystemExit(f"replicate process {r + 1} failed (exit {p.returncode})")
        line = [l for l in p.stdout.splitlines() if l.startswith("{")][-1]
        out.append(json.loads(line))
    return out


def graph_nodes(g, calls):
    """Nodes of a captured graph per captured call (hipGraphGetNodes on the
    graph torch captured), or None where the graph handle is not exposed."""
    import ctypes
    try:
        raw = g.raw_cuda_graph()
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(ctypes.c_void_p(raw), None, ctypes.byref(n)) != 0:
            return None
        return n.value / calls
    except Exception:  # noqa: BLE001 -- older torch, or a different runtime
        return None


def measure_latency(step, torch, a, w):
    """Per-call time of the search against the launch floor on the same
    stream: eager (one Python call per search, as the timed steps) and as a
    captured HIP graph of `steps` searches replayed as one launch; the floor
    is an empty kernel (one wave) launched the same ways.  The graph replay's
    output is checked against the eager output."""
    import ctypes
    from farthest_vector_search_amd.build import ROOF_LIB
    R = ctypes.CDLL(ROOF_LIB)
    R.vs_roof_empty.restype = ctypes.c_int32
    R.vs_roof_empty.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    K = a.steps
    res = {}

    def per_call_us(fn, reps=5):
        """Median over reps of (wall time of K back-to-back calls) / K."""
        vals = []
        fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            t0 = time.perf_counter()
            for _ in range(K):
                fn()
            torch.cuda.synchronize()
            vals.append((time.perf_counter() - t0) / K * 1e6)
        return sorted(vals)[len(vals) // 2]

    import farthest_vector_search_amd as vs
    dev = torch.device("cuda", torch.cuda.current_device())

    def empty():  # the stream handle taken the way the binding takes it
        if R.vs_roof_empty(1, vs._stream(dev)) != 0:
            raise RuntimeError("vs_roof_empty failed")

    res["eager_us_per_call"] = round(per_call_us(step), 2)
    res["eager_empty_kernel_us"] = round(per_call_us(empty), 2)
    res["eager_frac"] = round(res["eager_empty_kernel_us"] / res["eager_us_per_call"], 4)
    # graphs: K searches (or K empty kernels) captured once, replayed
    ref_idx = w["gpu_out"]["idx"].clone()
    ref_score = w["gpu_out"]["score"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    try:  # keep the captured graph so that its nodes can be counted
        g_search, kept = torch.cuda.CUDAGraph(keep_graph=True), True
    except TypeError:
        g_search, kept = torch.cuda.CUDAGraph(), False
    g_empty = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_search):
        for _ in range(K):
            step()
    res["graph_nodes_per_call"] = graph_nodes(g_search, K) if kept else None
    if kept:
        g_search.instantiate()
    with torch.cuda.graph(g_empty):
        for _ in range(K):
            empty()
    torch.cuda.synchronize()
    ok = True
    for _ in range(3):  # every replay checked against the eager result
        w["gpu_out"]["idx"].fill_(-1)
        g_search.replay()
        torch.cuda.synchronize()
        ok &= bool(torch.equal(w["gpu_out"]["idx"], ref_idx)
                   and torch.equal(w["gpu_out"]["score"].view(torch.int32),
                                   ref_score.view(torch.int32)))
    res["graph_us_per_call"] = round(per_call_us(g_search.replay) / K, 2)
    res["graph_empty_kernel_us"] = round(per_call_us(g_empty.replay) / K, 2)
    res["graph_frac"] = round(res["graph_empty_kernel_us"] / res["graph_us_per_call"], 4)
    res["graph_replays_match_eager"] = ok
    res["note"] = ("frac = empty-kernel time / search time per call on the same stream; "
                   f"{K} calls per timing, median of 5")
    return res


def main():
    a = parse()
    if a.traffic_from:
        record_traffic(a)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(queries split across GPUs with no exchange would be the way). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    replicas = []
    n_rep = 1 if (a.child or a.roof or a.copy_bytes > 0 or under_profiler()) else max(1, a.replicates)
    if n_rep > 1:
        replicas = run_replicates(a, n_rep)
    import torch
    import farthest_vector_search_amd as vs
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (gfx950) GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_bytes > 0:
        copy_calibration(a, torch)
        return
    if a.roof == "l2":
        measure_l2_roof(a, torch)
        return
    if a.roof == "mfma":
        measure_mfma_roof(a, torch)
        return
    if a.roof == "gather":
        measure_gather_roof(a, torch)
        return
    log(f"workload {a.workload}: generating inputs")
    if a.som:
        w, step, pairs, flops, launches_per_step, cfg = setup_som(a.workload, torch, vs, a)
    else:
        w, step, pairs, flops, launches_per_step, cfg = setup(a.workload, torch, vs, a)
    torch.cuda.synchronize()
    log(f"warmup {a.warmup} steps")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {a.steps} steps")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    with vs.KernelTimer(max_launches=a.steps * launches_per_step + 8) as kt:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(a.steps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / a.steps
    value = pairs * a.steps / dt
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps))
    # roofline of the dominant kernel: algorithmic work of the timed steps over
    # the summed durations of its launches (= per-launch work / mean launch time)
    launches = max(kt.launches, 1)
    kernel_ms = kt.ms / launches
    kernel_s_total = kt.ms * 1e-3
    if w["kind"] == "diversity" and a.div_mode == "gram":
        # the Gram scans are HBM-bound reads of one table row per sequence and
        # step (a run is one launch, or one per step for masks wider than the
        # whole-run kernel keeps): algorithmic bytes of the timed runs over
        # the dominant kernel's summed time
        achieved = w["run_bytes"] * a.steps / kernel_s_total / 1e9
        if a.div_ref == "centroid":
            # the running sums (120 MB) stream through HBM beside the Gram rows
            roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(achieved / PEAK_HBM_GBS, 4))
        else:
            roof = dict(bound="gather", achieved=round(achieved, 1), peak=PEAK_GRAM_GATHER_GBS,
                        unit="GB/s", frac=round(achieved / PEAK_GRAM_GATHER_GBS, 4),
                        frac_of_hbm_peak=round(achieved / PEAK_HBM_GBS, 4),
                        peak_source="measured: bench.py --roof gather (the run's own rows)")
    elif w["kind"] in ("dense", "diversity"):
        achieved = flops * a.steps / kernel_s_total / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_FP32_MFMA_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_FP32_MFMA_TFLOPS, 4))
    else:
        # sparse: 4 (fp32) or 2 (fp16 storage) codebook bytes per non-zero x
        # neuron multiply-add, served from the XCDs' L2 (each XCD's 4 MiB slice
        # is read from HBM once per round), so the roof is the measured
        # L2 -> CU bandwidth, not HBM
        achieved = w["value_bytes"] * w["nnz"] * w["nc"] * a.steps / kernel_s_total / 1e9
        roof = dict(bound="l2", achieved=round(achieved, 1), peak=PEAK_L2_WIDE_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_L2_WIDE_GBS, 4),
                    peak_source="measured: bench.py --roof l2, dwordx4_4x256B")
    roof["launches_per_step"] = launches // a.steps
    roof["kernel"] = kt.name
    roof["kernel_ms"] = round(kernel_ms, 5)
    # counters were taken for the default forms only
    other_form = (cfg.get("mode") in ("gram", "unfused") or cfg.get("reference") == "centroid"
                  or cfg.get("steps_per_run", w.get("steps")) != w.get("steps"))
    roof["traffic"] = (None if other_form else
                       load_traffic(a.traffic_json, DOMINANT[a.workload],
                                    cfg["workload"].replace("+som_epoch", "")))
    out = {
        "metric": METRIC, "value": value, "unit": "pairs/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": cfg, "roofline": roof,
        # HIP events between consecutive steps on the launch stream
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4),
                    "min": round(per_step[0], 4), "max": round(per_step[-1], 4)},
    }
    if replicas:
        vals = [r["value"] for r in replicas] + [value]
        med = sorted(vals)[len(vals) // 2]
        spread = (max(vals) - min(vals)) / med * 100.0
        out["replicates"] = {"processes": len(vals), "values": vals,
                             "ms_per_step": [r["ms_per_step"] for r in replicas] + [out["ms_per_step"]],
                             "spread_pct": round(spread, 3), "spread_within_1_5_pct": spread <= 1.5}
    if a.workload == 1 and not a.som and a.dense_mode == "fused":
        log("latency against the empty-kernel floor")
        out["latency"] = measure_latency(step, torch, a, w)
    if a.som:
        qe_final = float(w["som_qe"].cpu()[0])
        log("epoch phases")
        out["som_epoch"] = som_phase_times(w, torch)
        out["som_epoch"]["qe_last_epoch"] = qe_final
    if not a.no_cpu_baseline:
        log("cpu baseline (the oracle on the checked set) and parity of the timed output")
        if a.som:
            out["cpu_baseline"] = cpu_baseline_som(a.workload, w, a.cpu_seconds)
        else:
            out["cpu_baseline"], parity = cpu_baseline(a.workload, w, a.cpu_seconds)
            if parity is not None:
                out["parity"] = parity
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
