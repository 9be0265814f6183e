"""Pins for the oracle's segmented key layout (CPU only).

Ref2VA VSA, two-stage attention patch: the geometry mapper gives text,
reference-image and reference-audio tokens tiles of their own that stay dense,
and only generated-video key tiles are pruned.  Configure Sol Sparse Attention,
"The inputs that matter": a long reference video may be sparsified while
reference images and audio stay exact.  Segments start on key-block
boundaries; the rows from a segment's end to the next start are padding.
"""
import math

import numpy as np
import pytest

import workloads as W
from workloads import bf16_bits, bf16_to_f32, EXACT, CENTROID, DROP


def _small(**kw):
    args = dict(H=2, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=2, frame_tokens=320)
    args.update(kw)
    return W.ref2va_segments(**args)


def _q(orc, wl):
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, wl.kblock)
    return q8, qs, k8, ks


def _valid_rows(wl):
    ok = np.zeros(wl.Lkv, bool)
    for start, rows, _ in wl.segments:
        ok[start:start + rows] = True
    return ok


def test_prefix_layout_equals_two_segments(orc):
    """A dense prefix followed by one routed segment is the prefix layout."""
    wl = W.config(4, small=True)
    q8, qs, k8, ks = _q(orc, wl)
    P = wl.prefix_tokens
    kw = dict(v_bits=wl.v, tau=1.0, G=2, kblock=64)
    a = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, prefix=P, **kw)
    b = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, segments=[(0, P, 0), (P, wl.lkv_valid - P, 1)], **kw)
    for key in ("map", "kbar", "vbar", "count", "stats"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_hand_layout_states_and_counts(orc):
    """Text of 77 rows in a 192-row slot (blocks 0, 1 valid, block 2 padding
    only), an image of 100 rows at 192 (blocks 3, 4), video of 256 rows at 320
    (blocks 5..8, routed).  Dense blocks are exact, padding-only blocks
    dropped, counts are the valid rows (13 in block 1, 36 in block 4)."""
    d, H = 64, 1
    rng = np.random.default_rng(9)
    L = 640
    segs = [(0, 77, 0), (192, 100, 0), (320, 256, 1)]
    x = np.zeros((3, 1, H, L, d), np.float32)
    for start, rows, _ in segs:
        x[:, :, :, start:start + rows] = rng.standard_normal((3, 1, H, rows, d))
    q, k, v = (bf16_bits(t) for t in x)
    q8, qs = orc.quantize(q, 576, 128)
    k8, ks = orc.quantize(k, 576, 64)
    for G in (1, 2):
        r = orc.route(q8, k8, ks, 64, 576, 576, v_bits=v, tau=float("inf"), G=G, kblock=64, segments=segs)
        m = r["map"][0, 0]
        assert (m[:, [0, 1, 3, 4, 5, 6, 7, 8]] == EXACT).all()
        assert (m[:, [2, 9]] == DROP).all()
        n = r["count"][0, 0].sum(-1)
        assert n.tolist() == [64, 13, 0, 64, 36, 64, 64, 64, 64, 0]
        if G == 2:
            assert r["count"][0, 0, 1].tolist() == [13, 0] and r["count"][0, 0, 4].tolist() == [32, 4]
    # routing touches only blocks 5..8; at tau = -inf all of them become centroids
    r = orc.route(q8, k8, ks, 64, 576, 576, v_bits=v, tau=float("-inf"), G=1, kblock=64, segments=segs)
    m = r["map"][0, 0]
    assert (m[:, 5:9] == CENTROID).all() and (m[:, [0, 1, 3, 4]] == EXACT).all()


def test_all_exact_forward_is_softmax_over_valid_keys(orc):
    """With every block exact, the output is textbook softmax attention of the
    dequantized queries over exactly the valid key rows (padding excluded)."""
    wl = _small(H=1)
    q8, qs, k8, ks = _q(orc, wl)
    r = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=float("inf"), G=1, kblock=64,
                  segments=wl.segments)
    out, lse, sel = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                                vbar=r["vbar"], count=r["count"], v_bits=wl.v, kblock=64, G=1,
                                segments=wl.segments)
    ok = _valid_rows(wl)
    qd = q8[0, 0].astype(np.float64) * np.repeat(qs[0, 0].astype(np.float64), 128)[:, None]
    kd = k8[0, 0].astype(np.float64) * np.repeat(ks[0, 0].astype(np.float64), 64)[:, None]
    vd = bf16_to_f32(wl.v[0, 0]).astype(np.float64)
    x = qd[:wl.lq_valid] @ kd[ok].T / math.sqrt(wl.d)
    x -= x.max(axis=1, keepdims=True)
    p = np.exp(x)
    ref = (p / p.sum(axis=1, keepdims=True)) @ vd[ok]
    got = out.reshape(-1, wl.d)[:wl.lq_valid]
    assert np.abs(got - ref).max() < 1e-9


def test_padding_rows_of_v_do_not_matter(orc):
    wl = _small(H=1)
    q8, qs, k8, ks = _q(orc, wl)
    kw = dict(tau=1.0, G=2, kblock=64, segments=wl.segments)
    a = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, **kw)
    v2 = wl.v.copy()
    pad = ~_valid_rows(wl)
    v2[0, 0, pad] = bf16_bits(np.full((pad.sum(), wl.d), 7.5, np.float32))
    b = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=v2, **kw)
    assert np.array_equal(a["vbar"], b["vbar"]) and np.array_equal(a["map"], b["map"])
    fa = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, a["map"], kbar=a["kbar"], vbar=a["vbar"],
                     count=a["count"], v_bits=wl.v, kblock=64, G=2, segments=wl.segments)[0]
    fb = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, b["map"], kbar=b["kbar"], vbar=b["vbar"],
                     count=b["count"], v_bits=v2, kblock=64, G=2, segments=wl.segments)[0]
    assert np.array_equal(fa, fb)


def _brute_candidates_map(q8, qs, k8, ks, wl, tau):
    """Independent float64 threshold rule over an explicit candidate list: the
    routed key blocks with a valid row."""
    d = wl.d
    ok = _valid_rows(wl)
    nQB, nKB = wl.Lq // 128, wl.Lkv // 64
    routed = np.zeros(nKB, bool)
    for start, rows, rt in wl.segments:
        routed[start // 64:(start + max(rows, 1) + 63) // 64] = bool(rt)
    out = np.zeros((wl.H, nQB, nKB), np.uint8)
    near = np.zeros_like(out, bool)
    for h in range(wl.H):
        qd = q8[0, h].astype(np.float64) * np.repeat(qs[0, h].astype(np.float64), 128)[:, None]
        kd = k8[0, h].astype(np.float64) * np.repeat(ks[0, h].astype(np.float64), 64)[:, None]
        km = [kd[j * 64:(j + 1) * 64][ok[j * 64:(j + 1) * 64]].mean(0) if ok[j * 64:(j + 1) * 64].any() else None
              for j in range(nKB)]
        cand = [j for j in range(nKB) if km[j] is not None and routed[j]]
        for i in range(nQB):
            for j in range(nKB):
                out[h, i, j] = EXACT if km[j] is not None else DROP
            rows = slice(i * 128, min((i + 1) * 128, wl.lq_valid))
            if i * 128 >= wl.lq_valid:
                continue
            qm = qd[rows].mean(0)
            s = np.array([qm @ km[j] / math.sqrt(d) for j in cand])
            if s.std() == 0:
                continue
            z = (s - s.mean()) / s.std()
            for jj, j in enumerate(cand):
                near[h, i, j] = abs(z[jj] - tau) < 1e-9
                if z[jj] > tau:
                    out[h, i, j] = CENTROID
    return out, near


@pytest.mark.parametrize("sparse_ref_video", [True, False])
def test_threshold_rule_brute_force_over_routed_segments(orc, sparse_ref_video):
    wl = _small(sparse_reference_video=sparse_ref_video)
    q8, qs, k8, ks = _q(orc, wl)
    r = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=1.0, G=1, kblock=64,
                  segments=wl.segments)
    ref, near = _brute_candidates_map(q8, qs, k8, ks, wl, 1.0)
    assert not ((r["map"][0] != ref) & ~near).any()
    # dense segments exact whatever the rule
    ref_video = wl.segments[3]
    blocks = slice(ref_video[0] // 64, (ref_video[0] + ref_video[1] + 63) // 64)
    if not sparse_ref_video:
        assert (r["map"][..., blocks] == EXACT).all()
    assert (r["map"][..., :wl.segments[3][0] // 64] != CENTROID).all()


def test_topk_counts_with_segments(orc):
    wl = _small()
    q8, qs, k8, ks = _q(orc, wl)
    r = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, G=1, kblock=64, rule=1, sparsity=0.75,
                  segments=wl.segments)
    N = sum(-(-rows // 64) for start, rows, rt in wl.segments if rt)
    kept_routed = (r["map"][..., wl.segments[3][0] // 64:] == EXACT).sum(-1)
    assert (kept_routed == N - math.floor(0.75 * N)).all()


def test_segments_must_not_overlap_or_straddle(orc):
    wl = _small(H=1)
    q8, qs, k8, ks = _q(orc, wl)
    for bad in ([(0, 100, 0), (64, 100, 1)], [(0, 10, 0), (100, 50, 1)]):
        with pytest.raises(ValueError):
            orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=1.0, G=1, kblock=64,
                      segments=bad)
