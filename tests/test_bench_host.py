"""Host-side bench logic: the live-pair fraction behind the masked TFLOP/s figures."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import oracle  # noqa: E402


@pytest.mark.parametrize("Hg,Wg,M,s", [(64, 64, 32, 16), (128, 128, 32, 16), (32, 48, 16, 8), (24, 16, 8, 3),
                                       (16, 16, 8, 0), (12, 20, 4, 1)])
def test_live_fraction_matches_label_pairs(Hg, Wg, M, s):
    # brute force over the oracle's region labels: same-label (query, key) pairs per window
    lab = oracle.wattn_ref.region_labels(Hg, Wg, M, s).reshape(-1, M * M)
    live = (lab[:, :, None] == lab[:, None, :]).mean()
    assert bench.live_fraction(Hg, Wg, M, s) == pytest.approx(float(live), rel=1e-12)


def test_live_fraction_known_values():
    # one split axis of four windows at M = 32, s = 16: ((3 + 1/2) / 4)^2; two windows per axis: (3/4)^2
    assert bench.live_fraction(128, 128, 32, 16) == pytest.approx(0.765625)
    assert bench.live_fraction(64, 64, 32, 16) == pytest.approx(0.5625)
    assert bench.live_fraction(64, 64, 32, 0) == 1.0


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
