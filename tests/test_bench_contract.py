"""The benchmark's command-line contract that needs no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N with N > 1 exits with code 2 and
    says so, before it imports torch or touches a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_sparse_pair_count_matches_brute_force():
    """The FLOP count of the block-sparse bench rows: (query, key) pairs the
    block mask and the causal mask leave, against an element-wise count."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench

    rng = np.random.default_rng(5)
    for n, causal in ((200, True), (200, False), (256, True), (130, True)):
        nb = -(-n // 64)
        for m in (rng.random((nb, nb)) < 0.5, np.ones((nb, nb)), bench.sparse_band_mask(nb, 2)):
            m = np.asarray(m, np.uint8)
            vis = m[np.arange(n)[:, None] // 64, np.arange(n)[None, :] // 64] != 0
            if causal:
                vis &= np.tri(n, dtype=bool)
            assert bench.sparse_visible_pairs(m, n, causal) == int(vis.sum())
