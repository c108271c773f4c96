"""Parsers for the text fixtures under tests/golden/ (no arithmetic)."""
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def _num(s):
    return math.nan if s == "nan" else float(s)


def hand_cases():
    cases, cur = [], None
    for line in _lines("hand_cases.txt"):
        key, *rest = line.split()
        if key == "case":
            cur = dict(name=rest[0], q=[], c=[], mask=[])
            cases.append(cur)
        elif key == "cite":
            cur["cite"] = rest[0]
        elif key == "metric":
            cur["metric"] = int(rest[0])
        elif key == "q":
            cur["q"].append([float(x) for x in rest])
        elif key == "c":
            cur["c"].append([float(x) for x in rest])
        elif key == "mask":
            cur["mask"] = [int(x) for x in rest]
        elif key == "expect_idx":
            cur["expect_idx"] = int(rest[0])
        elif key == "expect_value":
            cur["expect_value"] = _num(rest[0])
    for c in cases:
        c["Q"] = np.array(c["q"], np.float32)
        c["C"] = np.array(c["c"], np.float32)
        nc = c["C"].shape[0]
        W = (nc + 31) // 32
        m = np.zeros((c["Q"].shape[0], W), np.uint32)
        for j in c["mask"]:
            m[:, j // 32] |= np.uint32(1 << (j % 32))
        c["mask_words"] = m if c["mask"] else None
    return cases


def diversity_walk():
    out = dict(c=[])
    for line in _lines("diversity_walk.txt"):
        key, *rest = line.split()
        if key == "c":
            out["c"].append([float(x) for x in rest])
        elif key == "seed":
            out["seed"] = int(rest[0])
        elif key == "expect_picks":
            out["picks"] = [int(x) for x in rest]
        elif key == "expect_values":
            out["values"] = [_num(x) for x in rest]
    out["C"] = np.array(out["c"], np.float32)
    return out


def diversity_centroid():
    """The centroid-reference walk; vectors given by their angle in degrees."""
    out = dict(angles=[])
    for line in _lines("diversity_centroid.txt"):
        key, *rest = line.split()
        if key == "angle":
            out["angles"].append(float(rest[0]))
        elif key == "seed":
            out["seed"] = int(rest[0])
        elif key == "expect_picks":
            out["picks"] = [int(x) for x in rest]
        elif key == "expect_values":
            out["values"] = [_num(x) for x in rest]
    a = np.deg2rad(np.array(out["angles"]))
    out["C"] = np.stack([np.cos(a), np.sin(a)], axis=1).astype(np.float32)
    return out


def csr_cases():
    ct, rows = [], []
    for line in _lines("csr_cases.txt"):
        key, *rest = line.split()
        if key == "ct":
            ct.append([float(x) for x in rest])
        elif key == "row":
            kv = dict(x.split("=") for x in rest)
            rows.append(dict(
                metric=int(kv["metric"]),
                idx=[int(kv["idx"])] if "idx" in kv else [],
                val=[float(kv["val"])] if "val" in kv else [],
                expect_idx=int(kv["expect_idx"]),
                expect_value=_num(kv["expect_value"])))
    return np.array(ct, np.float32), rows


def tile_rule():
    out = []
    for line in _lines("tile_rule.txt"):
        cache, d, b, approx = line.split()
        out.append((int(cache), int(d), int(b), int(approx)))
    return out
