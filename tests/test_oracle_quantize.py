"""Pins for the oracle's per-block INT8 quantizer (CPU only).

Configure Sol Sparse Attention, "How it works": Q and K are prequantized to INT8
and the same codes feed the routing proxy and the exact path.  FlashVSR Kitchen
Sparse Attention, opening section: the K/V cache is INT8 in 128-row slabs.
"""
import os

import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_examples.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        vals, scale, codes = [p.strip() for p in line.split("|")]
        rows.append(([float(x) for x in vals.split()], float(scale), [int(x) for x in codes.split()]))
    return rows


@pytest.mark.parametrize("vals,scale,codes", _golden())
def test_hand_examples(orc, vals, scale, codes):
    x = bf16_bits(np.array(vals, dtype=np.float32)).reshape(1, 1, 1, -1)
    assert np.array_equal(bf16_to_f32(x).ravel(), np.array(vals, dtype=np.float32)), "fixture must be bf16-exact"
    q, s = orc.quantize(x, rows_per_block=128)
    assert s.ravel()[0] == np.float32(scale)
    assert q.ravel().tolist() == codes


def test_valid_len_excludes_pad_rows(orc):
    # Row 1 is padding: it must not set amax and must get code 0.
    x = bf16_bits(np.array([[1.0, -0.5], [100.0, 100.0]], dtype=np.float32)).reshape(1, 1, 2, 2)
    q, s = orc.quantize(x, valid_len=1, rows_per_block=128)
    assert s.ravel()[0] == np.float32(1.0) / np.float32(127.0)
    assert q.reshape(2, 2).tolist() == [[127, -64], [0, 0]]   # -63.5 -> -64 (even)


@pytest.mark.parametrize("R", [64, 128])
def test_bound_range_and_extremes(orc, R):
    rng = np.random.default_rng(7)
    x = bf16_bits(rng.standard_normal((1, 3, 5 * R + 17, 64), dtype=np.float32) * 3)
    L = x.shape[2]
    valid = L - 5
    q, s = orc.quantize(x, valid_len=valid, rows_per_block=R)
    xf = bf16_to_f32(x).astype(np.float64)
    assert q.min() >= -127 and q.max() <= 127
    for h in range(3):
        for blk in range(s.shape[2]):
            r0, r1 = blk * R, min(blk * R + R, valid)
            if r0 >= valid:
                assert s[0, h, blk] == 0 and not q[0, h, blk * R:(blk + 1) * R].any()
                continue
            xb = xf[0, h, r0:r1]
            amax = np.abs(xb).max()
            assert s[0, h, blk] == np.float32(np.float32(amax) / np.float32(127))
            # the block maximum lands on +-127
            assert np.abs(q[0, h, r0:r1]).max() == 127
            # rounding error at most half a step (plus the float32 step of 127/amax)
            err = np.abs(xb - q[0, h, r0:r1] * (amax / 127.0))
            assert err.max() <= 0.5 * amax / 127.0 * (1 + 1e-5)
    assert not q[0, :, valid:].any()
