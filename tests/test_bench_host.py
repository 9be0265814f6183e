"""Host-side checks of bench.py (CPU only): the one-GPU contract, the
algorithmic op count behind the roofline figure, and the rule that traffic
is reported only from a counter summary taken on the same kernel source."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_ops_hand_count():
    # one head, two query blocks, three key blocks; map: 1 exact, 2 centroid, 0 dropped
    bmap = np.array([[[[1, 2, 0], [2, 2, 1]]]], dtype=np.uint8)
    count = np.array([[[[64.0], [0.0], [10.0]]]], dtype=np.float32)   # [B,H,nKB,G]
    d = 128
    ops, tiles, cols = bench.fwd_algorithmic_ops(bmap, count, d)
    # exact: (0,0) and (1,2); centroid columns with a non-zero count: (1,0) only
    assert tiles == 2 and cols == 1
    qk_tile = 2 * 128 * 64 * d          # S = Q K^T on one 128 x 64 tile
    pv_tile = 2 * 128 * 64 * d          # O += P V
    col = 2 * 128 * d + 2 * 128 * d     # one centroid column: its logit and its value
    assert ops == 2 * (qk_tile + pv_tile) + 1 * col


def test_traffic_only_for_the_same_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# header\nhbm_bytes_per_launch = 12345\nkernel_hash = abc123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic("abc123") == 12345.0
    assert bench.read_traffic("other") is None
    f.write_text("kernel_hash = abc123\n")
    assert bench.read_traffic("abc123") is None
