"""The product path has no CPU fallback and never touches the oracle (no GPU needed).

* without libvs.so every entry point raises before doing anything;
* host (CPU) tensors are refused, not computed on the CPU;
* importing the package loads nothing from ``oracle/``, and no package
  source names it.
"""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import farthest_vector_search_amd as vs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "farthest_vector_search_amd")

torch = pytest.importorskip("torch")


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(vs, "LIB_PATH", str(tmp_path / "libvs.so"))
    monkeypatch.setattr(vs, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        vs.lib()
    Q = torch.zeros(4, 8)
    with pytest.raises(RuntimeError, match="missing"):
        vs.vs_bmu_search(Q, Q)
    with pytest.raises(RuntimeError, match="missing"):
        vs.vs_diversity_step(Q, torch.zeros(4, dtype=torch.int32),
                             torch.zeros(4, 1, dtype=torch.int32))


def test_host_tensors_are_refused():
    if not os.path.exists(vs.LIB_PATH):
        pytest.skip("libvs.so not built")
    Q = torch.from_numpy(np.ones((4, 8), np.float32))
    with pytest.raises(TypeError, match="CUDA"):
        vs.vs_bmu_search(Q, Q)
    with pytest.raises(TypeError, match="CUDA"):
        vs.vs_candidate_norms(Q)


def test_package_does_not_load_the_oracle():
    code = ("import sys; import farthest_vector_search_amd; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True,
                         text=True, check=True)
    assert out.stdout.strip() == "False"
    for name in os.listdir(PKG):
        if name.endswith(".py"):
            text = open(os.path.join(PKG, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), name
