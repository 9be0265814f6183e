"""Pins for the oracle's virtual-KV gather (CPU only).

Configure H3 Static Virtual KV, mode list: "conservative" materializes the exact
seven-slice K/V; "fast" builds each logical slice by reading a physical bf16
slice (one of two) named by a source map, applies that slice's temporal rotary
phase, and only materializes INT8 — with nothing approximated.
"""
import numpy as np

import workloads as W
from workloads import bf16_bits, bf16_to_f32


def _phys(seed=0, H=2, S=128, n_phys=2, d=64):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((1, H, S * n_phys, d), dtype=np.float32))


def test_zero_phase_is_plain_copy(orc):
    S, d = 128, 64
    kp = _phys(S=S, d=d)
    src = np.array([1, 0, 1, 1], np.int32)
    cos = np.ones((4, 8), np.float32)
    sin = np.zeros((4, 8), np.float32)
    kl = orc.materialize_virtual_k(kp, S, src, cos, sin, rot_offset=4)
    expect = np.concatenate([kp[:, :, s * S:(s + 1) * S] for s in src], axis=2)
    assert np.array_equal(kl, expect)
    k8, ks, vbs = orc.gather_virtual_kv(kp, S, src, cos, sin, rot_offset=4)
    q8, qs = orc.quantize(expect, rows_per_block=64)
    assert np.array_equal(k8, q8) and np.array_equal(ks, qs)


def test_quarter_turn_is_exact_pair_swap(orc):
    S, d = 64, 32
    kp = _phys(seed=1, S=S, d=d)
    src = np.array([0, 1], np.int32)
    cos = np.zeros((2, 4), np.float32)
    sin = np.ones((2, 4), np.float32)
    kl = orc.materialize_virtual_k(kp, S, src, cos, sin, rot_offset=2)
    x = bf16_to_f32(kp)
    y = bf16_to_f32(kl)
    for p in range(4):
        c0 = 2 + 2 * p
        assert np.array_equal(y[..., c0], -x[..., c0 + 1])       # y0 = -x1
        assert np.array_equal(y[..., c0 + 1], x[..., c0])        # y1 = x0
    untouched = [c for c in range(d) if not 2 <= c < 10]
    assert np.array_equal(y[..., untouched], x[..., untouched])


def test_rotation_preserves_pair_norms(orc):
    wl = W.virtual_kv_residual(H=2, rows_per_slice=128)
    kl = orc.materialize_virtual_k(wl.k, 128, wl.src_map, wl.rope_cos, wl.rope_sin, wl.rot_offset)
    S = 128
    x = bf16_to_f32(wl.k).astype(np.float64)
    y = bf16_to_f32(kl).astype(np.float64)
    for l, s in enumerate(wl.src_map):
        xs = x[:, :, s * S:(s + 1) * S, :wl.d_rot].reshape(2, S, -1, 2)
        ys = y[:, :, l * S:(l + 1) * S, :wl.d_rot].reshape(2, S, -1, 2)
        nx, ny = np.hypot(xs[..., 0], xs[..., 1]), np.hypot(ys[..., 0], ys[..., 1])
        assert np.all(np.abs(nx - ny) <= 2 ** -7 * nx + 1e-30)
        # and the angle actually advanced by l * theta_p (checked on pairs with a sizeable norm)
        ang = np.angle(ys[..., 0] + 1j * ys[..., 1]) - np.angle(xs[..., 0] + 1j * xs[..., 1])
        theta = l * 10000.0 ** (-2.0 * np.arange(wl.d_rot // 2) / wl.d_rot)
        diff = np.angle(np.exp(1j * (ang - theta)))
        big = nx > 0.5
        assert np.abs(diff[big]).max() < 2e-2


def test_fast_equals_conservative(orc):
    wl = W.virtual_kv_residual(H=2, rows_per_slice=256)
    kl = orc.materialize_virtual_k(wl.k, 256, wl.src_map, wl.rope_cos, wl.rope_sin)
    q8, qs = orc.quantize(kl, rows_per_block=64)
    k8, ks, vbs = orc.gather_virtual_kv(wl.k, 256, wl.src_map, wl.rope_cos, wl.rope_sin)
    assert np.array_equal(k8, q8) and np.array_equal(ks, qs)


def test_v_block_source_table(orc):
    kp = _phys(S=128, d=64)
    src = np.array([0, 1, 1, 0], np.int32)
    _, _, vbs = orc.gather_virtual_kv(kp, 128, src, np.ones((4, 2), np.float32), np.zeros((4, 2), np.float32))
    assert vbs.tolist() == [0, 1, 2, 3, 2, 3, 0, 1]
