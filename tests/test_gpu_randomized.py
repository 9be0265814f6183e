"""Seeded randomized GPU parity: combinations of head size, key-block size,
centroid groups, routing rule, segmented key layouts with padding, valid
lengths and the floating QK path, of the INT8 K/V cache path (rules or
explicit maps) and of virtual K/V, each checked against the oracle to the same bars as the
hand-picked cases."""
import numpy as np
import pytest

import workloads as W
from workloads import CENTROID, DROP, EXACT
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
    """Odd seeds let the route sum the codes itself; even ones hand it the
    quantizer's column sums."""
    wl = random_case(seed)
    _check_workload(orc, wl, sums=seed % 2 == 0)


@pytest.mark.parametrize("seed", range(2000, 2064))
def test_random_configuration_medium(sa, orc, seed):
    """Segments of up to 12 key blocks (up to ~6K keys): several rounds
    of workgroups, longer tile lists and their ragged ends."""
    wl = random_case(seed, max_blocks=12)
    _check_workload(orc, wl, sums=seed % 2 == 1)


def random_int8v_case(seed: int) -> W.Workload:
    """K and V as an INT8 cache (FlashVSR Kitchen Sparse Attention, opening
    section): random head size, key-block size, V scale rows, ragged valid
    lengths, and either a routing rule or an explicit EXACT / CENTROID / DROP
    map (where K may carry one scale per 64 rows under 128-key blocks)."""
    rng = np.random.default_rng(5000 + seed)
    d = int(rng.choice([64, 128]))
    kblock = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 4))
    L = 128 * int(rng.integers(2, 17))
    lkv_valid = int(rng.integers(L // 2, L + 1))
    lq_valid = int(rng.choice([L, int(rng.integers(1, L + 1))]))
    mode = int(rng.integers(0, 3))            # 0 threshold, 1 fixed sparsity, 2 explicit map
    G = int(rng.integers(1, 3)) if mode == 0 else int(rng.integers(0, 3))
    q = W.iid_normal_bf16(rng, (1, H, L, d))
    k = W.iid_normal_bf16(rng, (1, H, L, d))
    v = W.iid_normal_bf16(rng, (1, H, L, d))
    for t in (k, v):
        t[0, :, lkv_valid:] = 0
    q[0, :, lq_valid:] = 0
    ksr = kblock if mode < 2 else int(rng.choice([64, kblock]))
    wl = W.Workload(f"random_int8v_{seed}", 1, H, L, L, d, lq_valid, lkv_valid, q, k, v,
                    threshold=float(rng.uniform(-0.5, 1.5)), centroids_per_block=G, kblock=kblock,
                    k_scale_rows=ksr, v_int8=True, v_scale_rows=int(rng.choice([64, 128])))
    if mode == 1:
        wl.rule, wl.sparsity = 1, float(rng.choice([0.0, 0.5, 0.75, 1.0]))
    elif mode == 2:
        states = np.array([EXACT, CENTROID, DROP] if G > 0 else [EXACT, DROP], np.uint8)
        wl.explicit_map = rng.choice(states, size=(1, H, L // 128, L // kblock))
        wl.map_kblock = kblock
        wl.threshold = float("nan")
    return wl


@pytest.mark.parametrize("seed", range(96))
def test_random_int8_cache_configuration(sa, orc, seed):
    wl = random_int8v_case(seed)
    _check_workload(orc, wl, sums=seed % 2 == 0)


def random_virtual_case(seed: int) -> W.Workload:
    """Virtual K/V (Configure H3 Static Virtual KV, mode list): logical slices
    gathered from random physical ones with temporal RoPE on a random even
    channel span; then an explicit map, the Sol rule or fixed sparsity over
    the logical keys, with bf16 or INT8 V read through the V block table."""
    rng = np.random.default_rng(7000 + seed)
    d = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 4))
    S = 128 * int(rng.integers(1, 5))                 # rows per slice
    n_phys = int(rng.integers(1, 4))
    n_logical = int(rng.integers(max(n_phys, 2), 8))
    src = rng.integers(0, n_phys, n_logical).astype(np.int32)
    rot_offset = 2 * int(rng.integers(0, d // 4))
    d_rot = 2 * int(rng.integers(1, (d - rot_offset) // 2 + 1))
    cos, sin = W.rope_tables(n_logical, d_rot)
    Lq = 128 * int(rng.integers(1, n_phys * S // 128 + 1))
    Lkv = n_logical * S
    q = W.iid_normal_bf16(rng, (1, H, Lq, d))
    k = W.iid_normal_bf16(rng, (1, H, n_phys * S, d))
    v = W.iid_normal_bf16(rng, (1, H, n_phys * S, d))
    mode = int(rng.integers(0, 3))                    # 0 explicit map, 1 threshold, 2 fixed sparsity
    G = int(rng.integers(0 if mode != 1 else 1, 3))
    wl = W.Workload(f"random_virtual_{seed}", 1, H, Lq, Lkv, d, Lq, Lkv, q, k, v,
                    threshold=float(rng.uniform(-0.5, 1.5)), centroids_per_block=G, kblock=64, k_scale_rows=64,
                    virtual=True, rows_per_slice=S, n_phys=n_phys, src_map=src, rope_cos=cos, rope_sin=sin,
                    rot_offset=rot_offset, d_rot=d_rot)
    wl.v_int8, wl.v_scale_rows = bool(rng.integers(0, 2)), 128
    if mode == 0:
        states = np.array([EXACT, CENTROID, DROP] if G > 0 else [EXACT, DROP], np.uint8)
        wl.explicit_map = rng.choice(states, size=(1, H, Lq // 128, Lkv // 64))
        wl.threshold = float("nan")
    elif mode == 2:
        wl.rule, wl.sparsity = 1, float(rng.choice([0.0, 0.5, 0.75, 1.0]))
    return wl


@pytest.mark.parametrize("seed", range(64))
def test_random_virtual_configuration(sa, orc, seed):
    wl = random_virtual_case(seed)
    _check_workload(orc, wl, sums=seed % 2 == 0)
