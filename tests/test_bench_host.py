"""Host-side pins of the benchmark's work count and command line (no GPU).

Throughput is algorithmic work: 14 D flop per visible (query, key) pair for
forward plus backward (4 D forward: Q K^T and P V; 10 D backward: the Q K^T
recompute, dV, dP, dK, dQ), counted over visible pairs only.  The pair counts
here are checked against closed forms and against a brute-force count of the
mask, so a wrong window boundary or a causal off-by-one fails.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(S, causal, window, seg=None):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    vis = np.ones((S, S), bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= (i - j < window) if causal else (np.abs(i - j) < window)
    if seg is not None:
        vis &= seg[:, None] == seg[None, :]
    return int(vis.sum())


@pytest.mark.parametrize("S,causal,window", [(1, True, 0), (7, True, 0), (64, True, 3), (100, True, 100),
                                             (37, False, 0), (129, True, 16)])
def test_visible_pairs_match_a_brute_force_count(S, causal, window):
    w = SimpleNamespace(S=S, B=2, window=window, causal=causal)
    assert bench.visible_pairs(w) == 2 * brute_pairs(S, causal, window)


def test_visible_pairs_of_packed_segments():
    seg = np.array([[0] * 5 + [1] * 9 + [2] * 3, [0] * 17], np.int32)
    w = SimpleNamespace(S=17, B=2, window=0, causal=True)
    want = brute_pairs(17, True, 0, seg[0]) + brute_pairs(17, True, 0, seg[1])
    assert bench.visible_pairs(w, seg) == want == (15 + 45 + 6) + 153


def test_closed_forms_of_the_measured_workloads():
    # causal: S (S + 1) / 2 per head; window W at S = 8192: W (W + 1) / 2 + (S - W) W
    causal = bench.workload("causal_gqa")
    assert bench.visible_pairs(causal) == causal.B * 4096 * 4097 // 2
    win = bench.workload("window_d512")
    assert bench.visible_pairs(win) == win.B * (1024 * 1025 // 2 + (8192 - 1024) * 1024) == 7_864_832
    # 14 D flop per pair, all query heads: 1.925 TFLOP per step at B=4, Hq=32, D=128
    flop = 14.0 * causal.D * bench.visible_pairs(causal) * causal.Hq
    assert flop == 1924615110656.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
