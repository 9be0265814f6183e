"""Pins for the oracle's virtual-V read (CPU only).

Configure H3 Static Virtual KV, mode list: the logical K/V context of seven
slices is re-read from two physical slices through a source map; "fast" only
materializes the INT8 keys, and "residual" keeps the real slices exact while
the virtual ones enter the same softmax as centroids.  The oracle reads V
through a table of logical 64-row blocks (v_block_src) instead of copying it.
These tests materialize the logical V independently (numpy concatenation of
the physical slices in source-map order) and hold the oracle's route and
forward, read through the table, to the results on the materialized V.
"""
import math

import numpy as np
import torch

import workloads as W
from workloads import bf16_bits, bf16_to_f32, CENTROID, DROP, EXACT


def _case(seed=40, H=2, S=128, n_phys=2, src=(0, 1, 1, 0, 1), d=64, d_rot=16, Lq=256):
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng.standard_normal((1, H, Lq, d), dtype=np.float32))
    kp = bf16_bits(rng.standard_normal((1, H, n_phys * S, d), dtype=np.float32))
    vp = bf16_bits(rng.standard_normal((1, H, n_phys * S, d), dtype=np.float32))
    src = np.asarray(src, dtype=np.int32)
    cos, sin = W.rope_tables(len(src), d_rot)
    return q, kp, vp, src, cos, sin


def _materialize_v(vp, S, src):
    """Logical V: physical slice src[l] for each logical slice l, concatenated."""
    return np.ascontiguousarray(np.concatenate([vp[:, :, s * S:(s + 1) * S] for s in src], axis=2))


def _deq(codes, scales, rows):
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), rows, axis=-1)[..., None]


def test_table_names_the_source_slice_blocks(orc):
    q, kp, vp, src, cos, sin = _case()
    _, _, vbs = orc.gather_virtual_kv(kp, 128, src, cos, sin)
    vl = _materialize_v(vp, 128, src)
    # row r of the logical V is row vbs[r // 64] * 64 + r % 64 of the physical V
    rows = vbs.astype(np.int64).repeat(64) * 64 + np.tile(np.arange(64), len(vbs))
    assert np.array_equal(vp[:, :, rows], vl)


def test_all_exact_through_table_is_sdpa_on_materialized_v(orc):
    S = 128
    q, kp, vp, src, cos, sin = _case()
    H, d = q.shape[1], q.shape[3]
    Lq, Lkv = q.shape[2], len(src) * S
    q8, qs = orc.quantize(q, Lq, 128)
    k8, ks, vbs = orc.gather_virtual_kv(kp, S, src, cos, sin)
    r = orc.route(q8, k8, ks, 64, Lq, Lkv, v_bits=vp, v_block_src=vbs, tau=float("inf"), G=1)
    assert (r["map"] == EXACT).all()
    out, lse, _ = orc.forward(q8, qs, k8, ks, 64, Lq, Lkv, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                              count=r["count"], v_bits=vp, v_block_src=vbs)
    vl = bf16_to_f32(_materialize_v(vp, S, src))[0].astype(np.float64)
    qd, kd = _deq(q8, qs, 128)[0], _deq(k8, ks, 64)[0]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    ref = torch.nn.functional.scaled_dot_product_attention(t(qd), t(kd), t(vl)).numpy()
    got = out.reshape(H, Lq, d)
    assert np.abs(got - ref).max() < 1e-12
    logits = np.einsum("hqd,hkd->hqk", qd, kd) / math.sqrt(d)
    ref_lse = torch.logsumexp(torch.from_numpy(logits), dim=-1).numpy()
    assert np.abs(lse.reshape(H, Lq) - ref_lse).max() < 1e-10


def test_centroids_through_table_are_means_of_materialized_v(orc):
    S = 128
    q, kp, vp, src, cos, sin = _case(seed=41)
    Lq, Lkv = q.shape[2], len(src) * S
    q8, qs = orc.quantize(q, Lq, 128)
    k8, ks, vbs = orc.gather_virtual_kv(kp, S, src, cos, sin)
    vl = bf16_to_f32(_materialize_v(vp, S, src)).astype(np.float64)
    for G in (1, 2):
        r = orc.route(q8, k8, ks, 64, Lq, Lkv, v_bits=vp, v_block_src=vbs, tau=0.5, G=G)
        gr = 64 // G
        ref = vl.reshape(1, q.shape[1], Lkv // gr, gr, -1).mean(axis=3).reshape(r["vbar"].shape)
        assert np.abs(r["vbar"] - ref).max() < 1e-12
        # the route on the materialized V gives the same map, centroids and statistics
        r2 = orc.route(q8, k8, ks, 64, Lq, Lkv, v_bits=_materialize_v(vp, S, src), tau=0.5, G=G)
        assert np.array_equal(r["map"], r2["map"]) and np.array_equal(r["vbar"], r2["vbar"])
        assert np.array_equal(r["kbar"], r2["kbar"]) and np.array_equal(r["count"], r2["count"])


def test_int8_v_through_table_equals_materialized_int8_v(orc):
    """INT8 V read through the table with 64- and 128-row physical scales
    against a materialized INT8 V whose 64-row blocks (codes and the scale that
    covers them) are copied from the physical blocks the table names."""
    S = 128
    q, kp, vp, src, cos, sin = _case(seed=42)
    H = q.shape[1]
    Lq, Lkv = q.shape[2], len(src) * S
    q8, qs = orc.quantize(q, Lq, 128)
    k8, ks, vbs = orc.gather_virtual_kv(kp, S, src, cos, sin)
    rng = np.random.default_rng(7)
    em = rng.choice(np.array([EXACT, CENTROID, DROP], np.uint8), size=(1, H, Lq // 128, Lkv // 64), p=[.5, .4, .1])
    for vrows in (64, 128):
        v8p, vsp = orc.quantize(vp, None, vrows)
        # materialize: logical block j <- physical block vbs[j]; its scale is the
        # physical scale covering that block
        v8l = np.concatenate([v8p[:, :, p * 64:(p + 1) * 64] for p in vbs], axis=2)
        vsl = np.stack([vsp[:, :, p * 64 // vrows] for p in vbs], axis=2)
        assert v8l.shape[2] == Lkv and not np.array_equal(vbs, np.arange(len(vbs)))
        for G in (1, 2):
            kw = dict(G=G, kblock=64, explicit_map=em, map_kblock=64)
            r1 = orc.route(q8, k8, ks, 64, Lq, Lkv, v8=v8p, v_scale=vsp, v_scale_rows=vrows, v_block_src=vbs, **kw)
            r2 = orc.route(q8, k8, ks, 64, Lq, Lkv, v8=v8l, v_scale=vsl, v_scale_rows=64, **kw)
            assert np.array_equal(r1["vbar"], r2["vbar"]) and np.array_equal(r1["map"], r2["map"])
            ref = _deq(v8l, vsl, 64).reshape(1, H, Lkv // (64 // G), 64 // G, -1).mean(axis=3)
            assert np.abs(r1["vbar"] - ref.reshape(r1["vbar"].shape)).max() < 1e-12
            fk = dict(kbar=r1["kbar"], vbar=r1["vbar"], count=r1["count"], kblock=64, G=G)
            o1, l1, _ = orc.forward(q8, qs, k8, ks, 64, Lq, Lkv, r1["map"], v8=v8p, v_scale=vsp,
                                    v_scale_rows=vrows, v_block_src=vbs, **fk)
            o2, l2, _ = orc.forward(q8, qs, k8, ks, 64, Lq, Lkv, r1["map"], v8=v8l, v_scale=vsl,
                                    v_scale_rows=64, **fk)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
