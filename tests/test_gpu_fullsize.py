"""GPU parity at the workloads' full sizes.

Codes, scales, tables, block maps and centroids are compared in full; outputs
are compared on every query block for the tiny Sol, FlashVSR LCSA and virtual-KV
workloads, and on sampled query blocks that the oracle computes one by one
(first and last blocks of each head, the blocks around the end of the valid
tokens, frame boundaries, and a seeded random set) for the 32K-token ones.  The launch configuration is the one bench.py times
(one call per entry point on the current stream); the measured workload is also
checked with bf16 output, as bench.py runs it.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import say
from tests.test_gpu_parity import _check_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import block_sparse_int8_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.device_check(torch.cuda.current_device())
    return m


def _sample(wl, n_random, seed, frame_tokens=None, prefix=0):
    nQB = wl.Lq // 128
    ids = set()
    for bh in (0, wl.B * wl.H - 1):
        for i in (0, 1, nQB - 2, nQB - 1):
            ids.add(bh * nQB + i)
        last_valid = (wl.lq_valid - 1) // 128
        ids.add(bh * nQB + last_valid)
        if frame_tokens:
            for f in range(1, 4):
                ids.add(bh * nQB + min(nQB - 1, (prefix + f * frame_tokens) // 128))
        if prefix:
            ids.add(bh * nQB + prefix // 128 - 1)
            ids.add(bh * nQB + prefix // 128)
    rng = np.random.default_rng(seed)
    ids.update(rng.choice(wl.B * wl.H * nQB, size=n_random, replace=False).tolist())
    return np.array(sorted(ids), dtype=np.int64)


def test_full_tiny_sol(sa, orc):
    _check_workload(orc, W.config(1))


def test_full_flashvsr_lcsa(sa, orc):
    wl = W.config(2)
    g, o = _check_workload(orc, wl)          # every query block
    per_head = (g["map"] == 1).reshape(wl.H, -1).sum(1) // 1
    # 128-key logical blocks: 518 exact per head (FlashVSR LCSA geometry)
    assert per_head.tolist() == [518] * wl.H


def test_full_wan14b_like(sa, orc):
    wl = W.config(3)
    sel = _sample(wl, 24, 3, frame_tokens=30 * 52)
    say(f"sampled {len(sel)} query blocks")
    g, o = _check_workload(orc, wl, sel=sel)
    kept = (g["map"][..., :-(-wl.lkv_valid // 64)] == 1).mean()
    say(f"kept fraction {kept:.4f}")
    # bench.py's configuration: bf16 output
    _check_workload(orc, wl, sel=sel[:12], out_dtype=torch.bfloat16)


def test_full_sol_prefix_2x32(sa, orc):
    wl = W.config(4)
    _check_workload(orc, wl, sel=_sample(wl, 24, 4, frame_tokens=84 * 48, prefix=1024))


def test_full_virtual_kv_residual(sa, orc):
    wl = W.config(5)
    _check_workload(orc, wl)                 # every query block (768)


def test_full_wan14b_like_topk(sa, orc):
    """Fixed-sparsity routing at 0.75 (Ref2VA VSA recipe) on the 32K workload:
    the whole map bit-exact, outputs on sampled query blocks."""
    wl = W.config(3)
    wl.rule, wl.sparsity = 1, 0.75
    g, o = _check_workload(orc, wl, sel=_sample(wl, 12, 6, frame_tokens=30 * 52))
    nvalid = -(-wl.lkv_valid // 64)
    kept = (g["map"][..., :nvalid] == 1).sum(-1)
    assert (kept == nvalid - int(np.floor(0.75 * nvalid))).all()


def test_full_sol_prefix_topk_2x32(sa, orc):
    wl = W.config(4)
    wl.rule, wl.sparsity = 1, 0.6
    _check_workload(orc, wl, sel=_sample(wl, 12, 7, frame_tokens=84 * 48, prefix=1024))


def test_full_ref2va_segments(sa, orc):
    """Reference-conditioned layout at full size (H=24, 17664 rows): text,
    reference image and audio dense, reference and generated video routed."""
    wl = W.ref2va_segments()
    sel = _sample(wl, 12, 8)
    seg_q = sorted({int(s[0]) // 128 for s in wl.segments})
    nQB = wl.Lq // 128
    sel = np.unique(np.concatenate([sel, np.array(seg_q, dtype=np.int64), (wl.H - 1) * nQB + np.array(seg_q)]))
    _check_workload(orc, wl, sel=sel)


def test_full_wan14b_like_float_qk(sa, orc):
    """The 32K workload with the floating QK path (sampled query blocks)."""
    wl = W.config(3)
    wl.qk_float = True
    _check_workload(orc, wl, sel=_sample(wl, 8, 9, frame_tokens=30 * 52))


def test_full_ref2va_segments_topk(sa, orc):
    """The reference-conditioned layout under the fixed-sparsity rule (0.75, the
    Ref2VA VSA recipe): only the routed video segments are pruned."""
    wl = W.ref2va_segments()
    wl.rule, wl.sparsity = 1, 0.75
    g, o = _check_workload(orc, wl, sel=_sample(wl, 8, 10))
    first_routed = int(wl.segments[3][0]) // 64
    assert (g["map"][..., :first_routed] != 2).all()


def test_full_flashvsr_lcsa_float_qk(sa, orc):
    """FlashVSR's LCSA pattern on the floating QK path (bf16 K and V)."""
    wl = W.config(2)
    wl.v_int8 = False
    wl.qk_float = True
    _check_workload(orc, wl, sel=_sample(wl, 16, 11, frame_tokens=32 * 64))
