"""bench.py without a GPU: the one-GPU contract and the algorithmic work it
divides by (the stated per-step formulas, recomputed here by hand on the toy
tree)."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

from conftest import ROOT

import workloads as W


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_of_the_toy_step():
    """Toy tree parent [-1,0,0,1,1,2] (depths 0,1,1,2,2,2), fp32, Hq=Hkv=4,
    D=64, L=128, V=1000; rows 0, 1 and 2 have children."""
    w = W.make("toy")
    a_attn, f_attn, a_acc = _bench().algorithmic(w)
    n, L, H, D, e = 6, 128, 4, 64, 4
    assert a_attn == H * (L + n) * D * 2 * e + 2 * n * H * D * e + n * 1 * 8
    visible = sum(L + d + 1 for d in (0, 1, 1, 2, 2, 2))
    assert f_attn == H * D * 4 * visible
    assert a_acc == n * 1000 * 4 + 3 * 1000 * 4
    # deterministic children read no draft rows
    assert _bench().algorithmic(w, topk=True)[2] == n * 1000 * 4
    assert np.array_equal(w.parents, [-1, 0, 0, 1, 1, 2])
