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


def test_accept_bytes_count_the_rows_the_walk_can_need():
    """Toy tree: rows 0, 1 and 2 have children.  A walk ending at a leaf
    (path 0 -> 1 -> 3) adds that leaf's target row; one stopping at a node
    with children (path 0 -> 2 after rejecting 2's child) adds nothing."""
    import torch
    w = W.make("toy")
    bench = _bench()
    V = 1000
    path = torch.full((1, 9), -1, dtype=torch.int32)
    path[0, :3] = torch.tensor([0, 1, 3])
    assert bench.accept_bytes(w, False, path, torch.tensor([2])) == (3 + 3 + 1) * V * 4
    assert bench.accept_bytes(w, True, path, torch.tensor([2])) == (3 + 1) * V * 4
    path[0, :3] = torch.tensor([0, 2, -1])
    assert bench.accept_bytes(w, False, path, torch.tensor([1])) == (3 + 3) * V * 4
    # an abandoned request (accept_len -1) adds no leaf row
    assert bench.accept_bytes(w, False, path, torch.tensor([-1])) == (3 + 3) * V * 4
    f = bench.attn_plus_accept(10.0, 4.0, 6.0, 1e-3, 1e-3, 6)
    assert f["bytes"] == 14.0 and f["bytes_every_target_row"] == 16.0
    assert abs(f["hbm_frac"] * bench.HBM_PEAK_GBS * 1e9 * 2e-3 - 14.0) < 1e-9
