"""Seeded randomized GPU parity: combinations of head size, key-block size,
centroid groups, routing rule, segmented key layouts with padding, valid
lengths and the floating QK path, each checked against the oracle to the
same bars as the hand-picked cases."""
import numpy as np
import pytest

import workloads as W
from tests.test_gpu_parity import _check_workload, sa  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def random_case(seed: int, max_blocks: int = 5) -> W.Workload:
    """Segments of up to max_blocks key blocks each (1-4 of them)."""
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    kblock = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 4))
    rule = int(rng.integers(0, 2))
    G = int(rng.integers(0 if rule == 1 else 1, 3))
    qk_float = bool(rng.integers(0, 2))
    # key layout: 1-4 segments on key-block boundaries with random padding
    segs, cursor = [], 0
    for _ in range(int(rng.integers(1, 5))):
        rows = int(rng.integers(1, max_blocks * kblock))
        segs.append((cursor, rows, int(rng.integers(0, 2))))
        cursor += -(-rows // kblock) * kblock + kblock * int(rng.integers(0, 2))
    if not any(r for _, _, r in segs):
        segs[-1] = (segs[-1][0], segs[-1][1], 1)
    L = -(-cursor // 128) * 128 + 128 * int(rng.integers(0, 2))
    end = segs[-1][0] + segs[-1][1]
    valid = np.zeros(L, bool)
    for s0, rows, _ in segs:
        valid[s0:s0 + rows] = True
    q = W.iid_normal_bf16(rng, (1, H, L, d))
    k = W.iid_normal_bf16(rng, (1, H, L, d))
    v = W.iid_normal_bf16(rng, (1, H, L, d))
    for t in (k, v):
        t[0, :, ~valid] = 0            # padding rows hold zeros
    q[0, :, end:] = 0
    use_segments = len(segs) > 1 or segs[0][2] == 0 or bool(rng.integers(0, 2))
    wl = W.Workload(f"random_{seed}", 1, H, L, L, d, end, end, q, k, v, threshold=float(rng.uniform(-0.5, 1.5)),
                    centroids_per_block=G, kblock=kblock, k_scale_rows=kblock,
                    segments=np.array(segs, np.int32) if use_segments else None)
    if not use_segments:   # plain layout: everything valid up to the end
        wl.lkv_valid = end
    wl.rule, wl.sparsity = rule, float(rng.choice([0.0, 0.25, 0.5, 0.75, 0.9, 1.0]))
    wl.qk_float = qk_float
    return wl


@pytest.mark.parametrize("seed", range(576))
def test_random_configuration(sa, orc, seed):
    wl = random_case(seed)
    _check_workload(orc, wl)


@pytest.mark.parametrize("seed", range(2000, 2064))
def test_random_configuration_medium(sa, orc, seed):
    """Segments of up to 12 key blocks (up to ~6K keys): several rounds
    of workgroups, longer tile lists and their ragged ends."""
    wl = random_case(seed, max_blocks=12)
    _check_workload(orc, wl)
