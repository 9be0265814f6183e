"""Pins for the oracle's routing (CPU only).

Configure Sol Sparse Attention, "How it works": per 128-token query block each
64-token key block gets a proxy score from the INT8 Q/K; it is skipped (becomes a
centroid) when its score exceeds mean + routing_threshold * std over the query
block's candidates.  "The inputs that matter": threshold default 1.0, manual
prefix protection.  FlashVSR Sparge Attention, "How it works": routing on logical
blocks, then conversion to the kernel's block geometry.
"""
import math

import numpy as np
import pytest

import workloads as W
from workloads import bf16_bits, bf16_to_f32, EXACT, CENTROID, DROP


def _quantized(orc, wl):
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, wl.kblock)
    return q8, qs, k8, ks


def _route(orc, wl, q8, k8, ks, **kw):
    args = dict(v_bits=wl.v, tau=wl.threshold, G=wl.centroids_per_block, prefix=wl.prefix_tokens,
                kblock=wl.kblock)
    args.update(kw)
    return orc.route(q8, k8, ks, wl.kblock, wl.lq_valid, wl.lkv_valid, **args)


def _brute_map(q8, qs, k8, ks, lq_valid, lkv_valid, tau, prefix=0, kblock=64):
    """Independent float64 formulation: proxy = dot of the dequantized block
    means divided by sqrt(d); z = (proxy - mean) / population std over the
    candidates; centroid iff z > tau.  Returns (map, z)."""
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    nQB, nKB = Lq // 128, Lkv // kblock
    out = np.zeros((B, H, nQB, nKB), np.uint8)
    zs = np.full((B, H, nQB, nKB), np.nan)
    for b in range(B):
        for h in range(H):
            qd = q8[b, h].astype(np.float64) * np.repeat(qs[b, h].astype(np.float64), 128)[:, None]
            kd = k8[b, h].astype(np.float64) * np.repeat(ks[b, h].astype(np.float64), kblock)[:, None]
            qm = [qd[i * 128:min((i + 1) * 128, lq_valid)].mean(0) if i * 128 < lq_valid else None
                  for i in range(nQB)]
            km = [kd[j * kblock:min((j + 1) * kblock, lkv_valid)].mean(0) if j * kblock < lkv_valid else None
                  for j in range(nKB)]
            cand = [j for j in range(nKB) if km[j] is not None and j * kblock >= prefix]
            for i in range(nQB):
                for j in range(nKB):
                    out[b, h, i, j] = EXACT if km[j] is not None else DROP
                if qm[i] is None or not cand:
                    continue
                s = np.array([qm[i] @ km[j] / math.sqrt(d) for j in cand])
                mu, sd = s.mean(), s.std()
                if sd == 0:
                    continue
                z = (s - mu) / sd
                for jj, j in enumerate(cand):
                    zs[b, h, i, j] = z[jj]
                    if z[jj] > tau:
                        out[b, h, i, j] = CENTROID
    return out, zs


@pytest.mark.parametrize("tau", [1.0, 0.3, -0.5, 2.0])
def test_matches_float64_brute_force(orc, tau):
    wl = W.tiny_sol(seed=11, H=3, L=768, d=64, valid=700)
    q8, qs, k8, ks = _quantized(orc, wl)
    r = _route(orc, wl, q8, k8, ks, tau=tau)
    ref, z = _brute_map(q8, qs, k8, ks, wl.lq_valid, wl.lkv_valid, tau)
    near = np.abs(z - tau) < 1e-9
    mism = (r["map"] != ref) & ~near
    assert not mism.any(), f"{mism.sum()} decisions differ from the brute force"
    # the row with no valid queries still routes (query-side padding does not change key decisions)


def test_prefix_and_correlated_brute_force(orc):
    wl = W.config(4, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    r = _route(orc, wl, q8, k8, ks)
    ref, z = _brute_map(q8, qs, k8, ks, wl.lq_valid, wl.lkv_valid, 1.0, prefix=wl.prefix_tokens)
    near = np.abs(z - 1.0) < 1e-9
    assert not ((r["map"] != ref) & ~near).any()
    npre = wl.prefix_tokens // 64
    assert (r["map"][..., :npre] == EXACT).all()      # prefix keys always exact
    assert (r["map"][..., npre:] == CENTROID).any()


def _outlier_case(c_val=2.0):
    """One query block whose rows are all e0; four key blocks, three all zero and
    the last with k[0] = c on every row.  Proxies (0, 0, 0, s), so the outlier's
    z-score is sqrt(3) with the population std (1.5 with the sample std)."""
    d = 64
    q = np.zeros((1, 1, 128, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 256, d), np.float32)
    k[0, 0, 192:, 0] = c_val
    v = np.zeros((1, 1, 256, d), np.float32)
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


@pytest.mark.parametrize("tau,expect_last", [(1.0, CENTROID), (1.6, CENTROID), (1.75, EXACT), (2.0, EXACT)])
def test_outlier_closed_form(orc, tau, expect_last):
    qb, kb, vb = _outlier_case()
    q8, qs = orc.quantize(qb, rows_per_block=128)
    k8, ks = orc.quantize(kb, rows_per_block=64)
    r = orc.route(q8, k8, ks, 64, 128, 256, v_bits=vb, tau=tau, G=1, kblock=64)
    assert r["map"][0, 0, 0].tolist() == [EXACT, EXACT, EXACT, expect_last]
    mu, sd = r["stats"][0, 0, 0]
    s = float(r["stats"][0, 0, 0][0]) * 4
    assert math.isclose((s - mu) / sd, math.sqrt(3.0), rel_tol=1e-12)


def test_outlier_low_threshold_skips_everything(orc):
    qb, kb, vb = _outlier_case()
    q8, qs = orc.quantize(qb, rows_per_block=128)
    k8, ks = orc.quantize(kb, rows_per_block=64)
    # zero blocks have z = -1/sqrt(3) ~ -0.577
    r = orc.route(q8, k8, ks, 64, 128, 256, v_bits=vb, tau=-0.5, G=1, kblock=64)
    assert r["map"][0, 0, 0].tolist() == [EXACT, EXACT, EXACT, CENTROID]
    r = orc.route(q8, k8, ks, 64, 128, 256, v_bits=vb, tau=-0.6, G=1, kblock=64)
    assert r["map"][0, 0, 0].tolist() == [CENTROID] * 4


def test_infinite_thresholds(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    valid_blocks = -(-wl.lkv_valid // 64)
    r = _route(orc, wl, q8, k8, ks, tau=float("inf"))
    kept = (r["map"][..., :valid_blocks] == EXACT).mean()
    assert kept == 1.0
    assert (r["map"][..., valid_blocks:] == DROP).all()
    r = _route(orc, wl, q8, k8, ks, tau=float("-inf"))
    assert (r["map"][..., :valid_blocks] == CENTROID).all()


def test_nested_in_threshold(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    prev = None
    for tau in [-1.0, -0.2, 0.0, 0.5, 1.0, 1.5, 3.0]:
        cen = _route(orc, wl, q8, k8, ks, tau=tau)["map"] == CENTROID
        if prev is not None:
            assert not (cen & ~prev).any(), "raising the threshold must only remove centroids"
        prev = cen


def test_power_of_two_scaling_invariance(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    base = _route(orc, wl, q8, k8, ks)["map"]
    wl2 = W.config(3, small=True)
    wl2.q = bf16_bits(bf16_to_f32(wl.q) * 4.0)
    wl2.k = bf16_bits(bf16_to_f32(wl.k) * 0.5)
    q8b, qsb, k8b, ksb = _quantized(orc, wl2)
    assert np.array_equal(q8, q8b) and np.array_equal(k8, k8b)
    assert np.array_equal(_route(orc, wl2, q8b, k8b, ksb)["map"], base)


def test_1x64_and_2x32_route_identically(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    m1 = _route(orc, wl, q8, k8, ks, G=1)["map"]
    m2 = _route(orc, wl, q8, k8, ks, G=2)["map"]
    assert np.array_equal(m1, m2)


def test_lcsa_closed_form_count():
    # 4 frames x 16 in-frame blocks: frame 0 sees 74 (3+4+5*12+4+3) key blocks,
    # frames 1..3 see twice that, 518 per head.
    m = W.lcsa_map(1, 12, 4, 16)
    assert (m == EXACT).sum(axis=(2, 3)).tolist() == [[518] * 12]
    per_frame = (m[0, 0] == EXACT).reshape(4, 16, 64).sum(axis=(1, 2)).tolist()
    assert per_frame == [74, 148, 148, 148]


def test_explicit_map_expansion_and_sanitizing(orc):
    wl = W.config(2, small=True)
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, 128)
    em = wl.explicit_map.copy()
    em[0, 0, 0, 5] = 7                  # out-of-range value -> exact
    em[0, 1, 0, 6] = CENTROID           # centroid with G = 0 -> exact
    r128 = orc.route(q8, k8, ks, 128, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, G=0, kblock=128,
                     explicit_map=em, map_kblock=128)
    expect = np.where(em > 1, EXACT, em)
    assert np.array_equal(r128["map"], expect)
    r64 = orc.route(q8, k8, ks, 128, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, G=0, kblock=64,
                    explicit_map=em, map_kblock=128)
    assert np.array_equal(r64["map"], np.repeat(expect, 2, axis=3))


def test_empty_key_blocks_drop_and_ragged(orc):
    wl = W.tiny_sol(seed=5, H=1, L=512, d=64, valid=300)
    q8, qs, k8, ks = _quantized(orc, wl)
    m = _route(orc, wl, q8, k8, ks)["map"]
    assert (m[..., 5:] == DROP).all()      # key rows >= 320 are all padding
    assert (m[..., :5] != DROP).all()


# ---------------------------------------------------------------------------
# Fixed-sparsity rule (Ref2VA VSA, two-stage attention patch: top-k pruning of
# the generated-video key tiles only, at a set sparsity such as 0.75).
# ---------------------------------------------------------------------------

def _ordered_case():
    """One query block whose rows are all e0 and seven key blocks: block j has
    k[0] = c_j on every row (block 6 is padding).  Each proxy is then a positive
    multiple of c_j, so the ranking is the ranking of c."""
    d = 64
    c = [3.0, -1.0, 5.0, 2.0, 4.0, 0.5]
    q = np.zeros((1, 1, 128, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 448, d), np.float32)
    for j, cj in enumerate(c):
        k[0, 0, j * 64:(j + 1) * 64, 0] = cj
    v = np.zeros((1, 1, 448, d), np.float32)
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


@pytest.mark.parametrize("sparsity,G,prefix,expect", [
    # ranking by c: blocks 2, 4, 0, 3, 5, 1
    (0.5, 1, 0, [EXACT, CENTROID, EXACT, CENTROID, EXACT, CENTROID]),     # prune floor(3.0) = 3
    (0.7, 1, 0, [CENTROID, CENTROID, EXACT, CENTROID, EXACT, CENTROID]),  # prune floor(4.2) = 4
    (0.3, 1, 0, [EXACT, CENTROID, EXACT, EXACT, EXACT, EXACT]),           # prune floor(1.8) = 1
    (0.0, 1, 0, [EXACT] * 6),
    (1.0, 2, 0, [CENTROID] * 6),
    (0.5, 0, 0, [EXACT, DROP, EXACT, DROP, EXACT, DROP]),                 # no centroids: pruned blocks drop
    (0.5, 1, 64, [EXACT, CENTROID, EXACT, EXACT, EXACT, CENTROID]),       # block 0 exempt; 5 candidates, prune 2
])
def test_topk_hand_ordered(orc, sparsity, G, prefix, expect):
    qb, kb, vb = _ordered_case()
    q8, qs = orc.quantize(qb, rows_per_block=128)
    k8, ks = orc.quantize(kb, valid_len=384, rows_per_block=64)
    r = orc.route(q8, k8, ks, 64, 128, 384, v_bits=vb, G=G, kblock=64, prefix=prefix, rule=1,
                  sparsity=sparsity)
    assert r["map"][0, 0, 0].tolist() == expect + [DROP]
    assert np.isnan(r["stats"]).all()


def test_topk_equal_scores_keep_lower_index(orc):
    d = 64
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 256, d)).astype(np.float32)
    blk = rng.standard_normal((64, d)).astype(np.float32)
    k = np.tile(blk, (10, 1))[None, None].repeat(2, axis=1)
    v = rng.standard_normal((1, 2, 640, d)).astype(np.float32)
    q8, qs = orc.quantize(bf16_bits(q), rows_per_block=128)
    k8, ks = orc.quantize(bf16_bits(k), rows_per_block=64)
    r = orc.route(q8, k8, ks, 64, 256, 640, v_bits=bf16_bits(v), G=1, kblock=64, rule=1, sparsity=0.75)
    # 10 equal scores: prune floor(7.5) = 7, keep blocks 0..2
    assert (r["map"][..., :3] == EXACT).all() and (r["map"][..., 3:] == CENTROID).all()


def _brute_topk(q8, qs, k8, ks, lq_valid, lkv_valid, sparsity, prefix=0, kblock=64):
    """Independent float64 formulation: proxy = dot of the dequantized block
    means over sqrt(d); keep the N - floor(sparsity*N) largest (stable order).
    Returns (map, rows whose kept/pruned boundary is too close to call)."""
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    nQB, nKB = Lq // 128, Lkv // kblock
    out = np.zeros((B, H, nQB, nKB), np.uint8)
    close = np.zeros((B, H, nQB), bool)
    sp = float(np.float32(sparsity))
    for b in range(B):
        for h in range(H):
            qd = q8[b, h].astype(np.float64) * np.repeat(qs[b, h].astype(np.float64), 128)[:, None]
            kd = k8[b, h].astype(np.float64) * np.repeat(ks[b, h].astype(np.float64), kblock)[:, None]
            km = [kd[j * kblock:min((j + 1) * kblock, lkv_valid)].mean(0) if j * kblock < lkv_valid else None
                  for j in range(nKB)]
            cand = [j for j in range(nKB) if km[j] is not None and j * kblock >= prefix]
            for i in range(nQB):
                for j in range(nKB):
                    out[b, h, i, j] = EXACT if km[j] is not None else DROP
                if i * 128 >= lq_valid or not cand:
                    continue
                qm = qd[i * 128:min((i + 1) * 128, lq_valid)].mean(0)
                s = np.array([qm @ km[j] / math.sqrt(d) for j in cand])
                keep = len(cand) - int(math.floor(sp * len(cand)))
                order = np.argsort(-s, kind="stable")
                for r, jj in enumerate(order):
                    if r >= keep:
                        out[b, h, i, cand[jj]] = CENTROID
                if 0 < keep < len(cand):
                    a, c = s[order[keep - 1]], s[order[keep]]
                    close[b, h, i] = abs(a - c) <= 1e-9 * max(abs(a), abs(c), 1e-300)
    return out, close


@pytest.mark.parametrize("sparsity", [0.5, 0.75, 0.6])
def test_topk_matches_float64_brute_force(orc, sparsity):
    wl = W.tiny_sol(seed=12, H=3, L=768, d=64, valid=700)
    q8, qs, k8, ks = _quantized(orc, wl)
    r = _route(orc, wl, q8, k8, ks, rule=1, sparsity=sparsity)
    ref, close = _brute_topk(q8, qs, k8, ks, wl.lq_valid, wl.lkv_valid, sparsity)
    assert not close.all()
    rows = ~close
    assert np.array_equal(r["map"][rows], ref[rows])


def test_topk_prefix_brute_force(orc):
    wl = W.config(4, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    r = _route(orc, wl, q8, k8, ks, rule=1, sparsity=0.75)
    ref, close = _brute_topk(q8, qs, k8, ks, wl.lq_valid, wl.lkv_valid, 0.75, prefix=wl.prefix_tokens)
    assert np.array_equal(r["map"][~close], ref[~close])
    npre = wl.prefix_tokens // 64
    assert (r["map"][..., :npre] == EXACT).all()


def test_topk_counts_and_nesting(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    nvalid = -(-wl.lkv_valid // 64)
    prev = None
    for sp in [0.0, 0.25, 0.5, 0.7, 0.75, 0.9, 1.0]:
        m = _route(orc, wl, q8, k8, ks, rule=1, sparsity=sp)["map"]
        kept = (m[..., :nvalid] == EXACT).sum(axis=-1)
        assert (kept == nvalid - math.floor(float(np.float32(sp)) * nvalid)).all()
        assert (m[..., nvalid:] == DROP).all()
        ex = m == EXACT
        if prev is not None:
            assert not (ex & ~prev).any(), "raising the sparsity must only remove exact blocks"
        prev = ex


def test_topk_power_of_two_scaling_invariance(orc):
    wl = W.config(3, small=True)
    q8, qs, k8, ks = _quantized(orc, wl)
    base = _route(orc, wl, q8, k8, ks, rule=1, sparsity=0.75)["map"]
    wl2 = W.config(3, small=True)
    wl2.q = bf16_bits(bf16_to_f32(wl.q) * 2.0)
    wl2.k = bf16_bits(bf16_to_f32(wl.k) * 0.25)
    q8b, qsb, k8b, ksb = _quantized(orc, wl2)
    assert np.array_equal(_route(orc, wl2, q8b, k8b, ksb, rule=1, sparsity=0.75)["map"], base)


def test_topk_rejects_bad_sparsity(orc):
    wl = W.tiny_sol(seed=1, H=1, L=256, d=64)
    q8, qs, k8, ks = _quantized(orc, wl)
    for sp in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            _route(orc, wl, q8, k8, ks, rule=1, sparsity=sp)
