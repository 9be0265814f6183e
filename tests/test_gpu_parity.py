"""GPU parity: the HIP path (through the C ABI) against the oracle on the same
seeded inputs.  Every test here needs an MI355X."""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import bf16_bits, EXACT, CENTROID, DROP
from tests.helpers import (MAX_ABS, MEAN_ABS, bf16_dev, compare_maps, compare_outputs, gpu_pipeline, say,
                           tie_blocks)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import block_sparse_int8_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.device_check(torch.cuda.current_device())
    return m


def _check_workload(orc, wl, tau=None, sel=None, out_dtype=torch.float32, tol=(MAX_ABS, MEAN_ABS), sums=True):
    say(f"case {wl.name} H={wl.H} Lq={wl.Lq} Lkv={wl.Lkv} d={wl.d} tau={tau if tau is not None else wl.threshold} "
        f"sums={sums}")
    g = gpu_pipeline(wl, tau=tau, out_dtype=out_dtype, sums=sums)
    o = orc.run(wl, sel=sel, tau=tau)
    assert np.array_equal(g["q8"], o["q8"]) and np.array_equal(g["q_scale"], o["q_scale"]), "Q codes differ"
    assert np.array_equal(g["k8"], o["k8"]) and np.array_equal(g["k_scale"], o["k_scale"]), "K codes differ"
    if wl.virtual:
        assert np.array_equal(g["v_block_src"], o["v_block_src"])
    if wl.v_int8:
        assert np.array_equal(g["v8"], o["v8"]) and np.array_equal(g["v_scale"], o["v_scale"])
    bad, ties, tie_mism = compare_maps(g["map"], o["map"], o["tie"])
    say(f"  map: {g['map'].size} entries, exact {int((g['map'] == 1).sum())}, centroid "
        f"{int((g['map'] == 2).sum())}, ties {ties}, tie mismatches {tie_mism}")
    assert bad == 0, f"{bad} block decisions differ outside the tie band"
    G = wl.centroids_per_block
    if G > 0:
        assert np.array_equal(g["count"], o["count"].astype(np.float32))
        kerr = np.abs(g["kbar"] - o["kbar"]).max()
        verr = np.abs(g["vbar"] - o["vbar"]).max()
        assert kerr <= 1e-5 * max(1.0, np.abs(o["kbar"]).max()) and verr <= 1e-5 * max(1.0, np.abs(o["vbar"]).max())
    if wl.explicit_map is None:
        # statistics agree to float64 rounding of the sums
        st_ok = np.isfinite(o["stats"])
        assert np.allclose(g["stats"][st_ok], o["stats"][st_ok], rtol=1e-9, atol=0)
    nQB = wl.Lq // 128
    skip = tie_blocks(g["map"], o["map"], nQB)
    mx, mean, rows = compare_outputs(g["out"], o["out"], o["sel"], nQB, wl.Lq, wl.lq_valid, skip)
    say(f"  out: rows {rows}, max-abs {mx:.3e}, mean-abs {mean:.3e}, blocks skipped for ties {len(skip)}")
    assert mx <= tol[0] and mean <= tol[1]
    # lse on valid rows.  The kernel's row sum adds the bf16-rounded weights it
    # also uses for PV, each within 2^-9 (relative) of the exact weight, so
    # |lse - lse_exact| <= ln(1 + 2^-9) ~= 1.95e-3 plus fp32 rounding.
    B_H = wl.B * wl.H
    gl = g["lse"].reshape(B_H, wl.Lq)
    for e, sid in enumerate(np.asarray(o["sel"])):
        if int(sid) in skip:
            continue
        bh, i = divmod(int(sid), nQB)
        ol = o["lse"][e]
        fin = np.isfinite(ol)
        assert np.array_equal(np.isfinite(gl[bh, i * 128:(i + 1) * 128]), fin)
        if fin.any():
            assert np.abs(gl[bh, i * 128:(i + 1) * 128][fin] - ol[fin]).max() < 2.5e-3
    return g, o


def test_device_is_gfx950(sa):
    sa.device_check(0)
    say("library:", sa.library_path())


@pytest.mark.parametrize("d,R,L,valid", [(128, 128, 1024, 1000), (128, 64, 768, 768), (64, 128, 512, 3),
                                         (64, 64, 256, 0)])
def test_quantize_bitexact(sa, orc, d, R, L, valid):
    say(f"case quantize d={d} R={R} L={L} valid={valid}")
    rng = np.random.default_rng(d + R + L)
    x = rng.standard_normal((2, 3, L, d), dtype=np.float32) * rng.uniform(0.1, 10, (2, 3, 1, 1)).astype(np.float32)
    if L >= 2 * R:
        x[1, 2, R:2 * R] = 0.0        # an all-zero block
    xb = bf16_bits(x)
    g8, gs = sa.quantize_qk_int8(bf16_dev(xb), valid, R)
    o8, os_ = orc.quantize(xb, valid, R)
    assert np.array_equal(g8.cpu().numpy(), o8) and np.array_equal(gs.cpu().numpy(), os_)


def test_quantize_strided_view(sa, orc):
    say("case quantize strided")
    rng = np.random.default_rng(5)
    xb = bf16_bits(rng.standard_normal((2, 6, 512, 128), dtype=np.float32))
    full = bf16_dev(xb)
    view = full[:, 1::2]                       # stride over heads
    g8, gs = sa.quantize_qk_int8(view, 500, 128)
    o8, os_ = orc.quantize(np.ascontiguousarray(xb[:, 1::2]), 500, 128)
    assert np.array_equal(g8.cpu().numpy(), o8) and np.array_equal(gs.cpu().numpy(), os_)
    # [B,L,H,d] memory viewed as [B,H,L,d]
    blhd = bf16_dev(np.ascontiguousarray(xb.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    g8, gs = sa.quantize_qk_int8(blhd, 512, 64)
    o8, os_ = orc.quantize(xb, 512, 64)
    assert np.array_equal(g8.cpu().numpy(), o8) and np.array_equal(gs.cpu().numpy(), os_)


def test_gather_bitexact(sa, orc):
    wl = W.config(5, small=True)
    say(f"case gather {wl.name}")
    kq, ks, vbs = sa.gather_virtual_kv(bf16_dev(wl.k), wl.rows_per_slice, wl.src_map.tolist(),
                                       torch.from_numpy(wl.rope_cos).cuda(), torch.from_numpy(wl.rope_sin).cuda())
    o8, os_, ovbs = orc.gather_virtual_kv(wl.k, wl.rows_per_slice, wl.src_map, wl.rope_cos, wl.rope_sin)
    assert np.array_equal(kq.cpu().numpy(), o8)
    assert np.array_equal(ks.cpu().numpy(), os_)
    assert np.array_equal(vbs.cpu().numpy(), ovbs)
    # the conservative path: materialize then quantize, with the GPU quantizer
    kl = orc.materialize_virtual_k(wl.k, wl.rows_per_slice, wl.src_map, wl.rope_cos, wl.rope_sin)
    g8, gs = sa.quantize_qk_int8(bf16_dev(kl), kl.shape[2], 64)
    assert np.array_equal(g8.cpu().numpy(), kq.cpu().numpy()) and np.array_equal(gs.cpu().numpy(), ks.cpu().numpy())


def test_gather_batched(sa, orc):
    """Two batch entries of physical K through the same source map."""
    wl = W.config(5, small=True)
    rng = np.random.default_rng(97)
    k2 = np.concatenate([wl.k, W.iid_normal_bf16(rng, wl.k.shape)], axis=0)
    say(f"case gather batched B={k2.shape[0]}")
    kq, ks, vbs = sa.gather_virtual_kv(bf16_dev(k2), wl.rows_per_slice, wl.src_map.tolist(),
                                       torch.from_numpy(wl.rope_cos).cuda(), torch.from_numpy(wl.rope_sin).cuda())
    o8, os_, ovbs = orc.gather_virtual_kv(k2, wl.rows_per_slice, wl.src_map, wl.rope_cos, wl.rope_sin)
    assert kq.shape[0] == 2
    assert np.array_equal(kq.cpu().numpy(), o8) and np.array_equal(ks.cpu().numpy(), os_)
    assert np.array_equal(vbs.cpu().numpy(), ovbs)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_small(sa, orc, n):
    _check_workload(orc, W.config(n, small=True))


@pytest.mark.parametrize("tau", [float("inf"), float("-inf"), 0.0, 2.0])
def test_thresholds(sa, orc, tau):
    wl = W.config(3, small=True)
    g, o = _check_workload(orc, wl, tau=tau)
    valid_blocks = -(-wl.lkv_valid // 64)
    if tau == float("inf"):
        assert (g["map"][..., :valid_blocks] == EXACT).all()    # kept fraction 1.0
    if tau == float("-inf"):
        assert (g["map"][..., :valid_blocks] == CENTROID).all()


def test_2x32_routes_like_1x64(sa):
    wl = W.config(3, small=True)
    g1 = gpu_pipeline(wl, G=1)
    g2 = gpu_pipeline(wl, G=2)
    assert np.array_equal(g1["map"], g2["map"])


def test_d64_ragged_tiny(sa, orc):
    _check_workload(orc, W.tiny_sol(seed=9, H=3, L=640, d=64, valid=577, centroids_per_block=2), tau=0.5)


def test_all_exact_equals_dense_attention(sa, orc):
    """tau = +inf: every block exact, so the result is plain softmax attention on
    the dequantized INT8 Q/K (checked through the oracle, whose all-exact mode is
    pinned to library SDPA)."""
    _check_workload(orc, W.tiny_sol(seed=12, H=2, L=1024, d=128, valid=1000), tau=float("inf"))


def test_lcsa_map_expansion_invariance(sa):
    """A 128-key map expanded to 64-key physical blocks gives the same output as
    running on 128-key blocks (FlashVSR Sparge Attention, "How it works")."""
    wl = W.config(2, small=True)
    g128 = gpu_pipeline(wl)
    g64 = gpu_pipeline(wl, kblock=64, map_kblock=128)
    assert np.array_equal(np.repeat(g128["map"], 2, axis=3), g64["map"])
    assert np.abs(g128["out"] - g64["out"]).max() < 1e-6


def test_bf16_output(sa, orc):
    wl = W.config(1)
    g32 = gpu_pipeline(wl)
    g16 = gpu_pipeline(wl, out_dtype=torch.bfloat16)
    assert np.abs(g16["out"] - g32["out"]).max() <= 2 ** -8 * np.abs(g32["out"]).max() + 1e-6


def test_deterministic(sa):
    wl = W.config(4, small=True)
    a = gpu_pipeline(wl)
    b = gpu_pipeline(wl)
    for key in ("map", "kbar", "vbar", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key


def test_empty_and_degenerate(sa, orc):
    # nothing valid: zeros and lse = -inf everywhere
    wl = W.tiny_sol(seed=3, H=1, L=256, d=64, valid=0)
    g = gpu_pipeline(wl)
    assert not g["out"].any() and np.isneginf(g["lse"]).all()
    assert (g["map"] == DROP).all()
    # keys valid, queries not
    wl = W.tiny_sol(seed=4, H=1, L=256, d=64)
    wl.lq_valid = 0
    g = gpu_pipeline(wl)
    assert not g["out"].any()
    # a single valid key
    wl = W.tiny_sol(seed=4, H=1, L=256, d=64)
    wl.lkv_valid = 1
    _check_workload(orc, wl)


def test_centroid_only_row(sa, orc):
    """tau = -inf: every block a centroid; the output is a count-weighted
    softmax over centroids only."""
    _check_workload(orc, W.config(4, small=True), tau=float("-inf"))


@pytest.mark.parametrize("G", [1, 2])
def test_sol_kblock128(sa, orc, G):
    """Sol routing on 128-key blocks (one K scale per block): four 32-row chunks
    per block sum, and centroid groups of 128 or 2 x 64 rows."""
    wl = W.tiny_sol(seed=21, H=2, L=1024, d=128, valid=1000, centroids_per_block=G)
    wl.kblock = 128
    wl.k_scale_rows = 128
    _check_workload(orc, wl, tau=0.5)


def test_saturated_block_sums(sa, orc):
    """Blocks whose codes are all +-127 with one sign per column: query block sums
    and 128-key block sums reach +-127*128, the ends of the range the routing
    proxy's two-digit split must cover; the other blocks stay random so the
    proxy's spread is not degenerate."""
    wl = W.tiny_sol(seed=22, H=2, L=1024, d=128, centroids_per_block=1)
    wl.kblock = 128
    wl.k_scale_rows = 128
    rng = np.random.default_rng(23)
    q = np.ascontiguousarray(wl.q.copy())
    k = np.ascontiguousarray(wl.k.copy())
    one, minus_one = bf16_bits(np.float32(1.0)), bf16_bits(np.float32(-1.0))
    for h in range(wl.H):
        for blk in (0, 3, 6):
            signs = rng.integers(0, 2, size=wl.d).astype(bool)
            q[0, h, blk * 128:(blk + 1) * 128, :] = np.where(signs, one, minus_one)
            signs = rng.integers(0, 2, size=wl.d).astype(bool)
            k[0, h, blk * 128:(blk + 1) * 128, :] = np.where(signs, one, minus_one)
    wl.q, wl.k = q, k
    g, o = _check_workload(orc, wl, tau=0.5)
    # the saturated blocks really are at the extreme
    assert np.abs(o["q8"][0, 0, :128].astype(np.int32).sum(axis=0)).max() == 127 * 128
    assert np.abs(o["k8"][0, 0, 384:512].astype(np.int32).sum(axis=0)).max() == 127 * 128


@pytest.mark.parametrize("d,G,sparsity,kblock", [(128, 1, 0.75, 64), (128, 2, 0.5, 64), (64, 1, 0.6, 64),
                                                 (128, 0, 0.75, 64), (128, 1, 0.7, 128), (64, 1, 0.0, 64),
                                                 (128, 2, 1.0, 64)])
def test_topk_routing(sa, orc, d, G, sparsity, kblock):
    """Fixed-sparsity rule: bit-exact map (no tie band), then the forward pass
    over it; G = 0 drops the pruned blocks."""
    wl = W.tiny_sol(seed=31, H=2, L=1024, d=d, valid=1000, centroids_per_block=max(G, 1))
    wl.centroids_per_block = G
    wl.rule, wl.sparsity = 1, sparsity
    wl.kblock = wl.k_scale_rows = kblock
    g, o = _check_workload(orc, wl)
    assert np.isnan(g["stats"]).all()


def test_topk_equal_scores(sa, orc):
    """Identical key blocks give equal proxies: the kept blocks are the lowest
    indices, on the GPU as in the oracle."""
    wl = W.tiny_sol(seed=32, H=2, L=1024, d=128, centroids_per_block=1)
    k = wl.k.copy()
    k[:, :, :, :] = np.tile(k[:, :, :64, :], (1, 1, 16, 1))
    wl.k = k
    wl.rule, wl.sparsity = 1, 0.75
    g, o = _check_workload(orc, wl)
    assert (g["map"][..., :4] == 1).all() and (g["map"][..., 4:] == 2).all()


def test_topk_prefix(sa, orc):
    wl = W.config(4, small=True)
    wl.rule, wl.sparsity = 1, 0.75
    _check_workload(orc, wl)


def _segmented(**kw):
    args = dict(H=2, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=2, frame_tokens=320)
    args.update(kw)
    return W.ref2va_segments(**args)


@pytest.mark.parametrize("G,sparse_ref_video,kblock", [(1, True, 64), (2, False, 64), (1, True, 128)])
def test_segmented_layout_threshold(sa, orc, G, sparse_ref_video, kblock):
    """Dense text / image / audio segments, routed video segments, each padded
    to a key-block boundary: several masked tiles per query block."""
    wl = _segmented(centroids_per_block=G, sparse_reference_video=sparse_ref_video, kblock=kblock)
    g, o = _check_workload(orc, wl)
    first_routed = wl.segments[3][0] if sparse_ref_video else wl.segments[4][0]
    assert (g["map"][..., :first_routed // kblock] != 2).all()


@pytest.mark.parametrize("G", [1, 0])
def test_segmented_layout_topk(sa, orc, G):
    wl = _segmented(centroids_per_block=max(G, 1))
    wl.centroids_per_block = G
    wl.rule, wl.sparsity = 1, 0.75
    _check_workload(orc, wl)


@pytest.mark.parametrize("d,G,kblock,valid", [(128, 1, 64, 1000), (64, 1, 64, 1024), (128, 2, 64, 1000),
                                              (128, 1, 128, 1000)])
def test_float_qk_forward(sa, orc, d, G, kblock, valid):
    """Floating QK^T on the bf16 Q/K for the exact tiles; same map and
    centroids as the INT8 path."""
    wl = W.tiny_sol(seed=51, H=2, L=1024, d=d, valid=valid, centroids_per_block=G)
    wl.kblock = wl.k_scale_rows = kblock
    wl.qk_float = True
    _check_workload(orc, wl, tau=0.5)


@pytest.mark.parametrize("kblock,G,v_int8,d", [(64, 1, False, 128), (64, 0, False, 64), (128, 0, True, 128),
                                                (128, 2, False, 64)])
def test_exact_tile_counts(sa, orc, kblock, G, v_int8, d):
    """Explicit maps giving the query blocks 0..7 exact key blocks each (the
    rest centroids, or dropped without centroids): the forward's tile loop
    runs every small count of exact tiles, ends on both tile parities, and
    meets the tile holding the end of the valid keys (1000 of 1024)."""
    L, H = 1024, 2
    wl = W.tiny_sol(seed=61, H=H, L=L, d=d, valid=1000, centroids_per_block=G)
    wl.kblock = wl.k_scale_rows = wl.map_kblock = kblock
    if v_int8:
        wl.v_int8, wl.v_scale_rows = True, kblock
    nQB, nKB = L // 128, L // kblock
    rng = np.random.default_rng(62)
    em = np.full((1, H, nQB, nKB), CENTROID if G > 0 else DROP, np.uint8)
    for h in range(H):
        for i in range(nQB):
            n = (i + 3 * h) % 8
            em[0, h, i, rng.choice(nKB, size=n, replace=False)] = EXACT
    wl.explicit_map = em
    g, o = _check_workload(orc, wl)
    counts = (g["map"] == EXACT).sum(-1)
    assert set(counts.ravel().tolist()) == set(range(8))


def test_float_qk_prefix_and_segments(sa, orc):
    wl = W.config(4, small=True)
    wl.qk_float = True
    _check_workload(orc, wl)
    wl = _segmented(centroids_per_block=2)
    wl.qk_float = True
    _check_workload(orc, wl)


def test_float_qk_explicit_map_no_centroids(sa, orc):
    """The LCSA pattern over bf16 K/V (G = 0)."""
    wl = W.config(2, small=True)
    wl.v_int8 = False
    wl.qk_float = True
    _check_workload(orc, wl)


def test_float_qk_and_topk_degenerate(sa, orc):
    """Nothing valid on the floating path; a single valid key (floating path,
    and the fixed-sparsity rule with one candidate, floor(0.75) = 0 pruned);
    a sparsity that prunes all but one of five candidates."""
    wl = W.tiny_sol(seed=5, H=1, L=256, d=64, valid=0)
    wl.qk_float = True
    g = gpu_pipeline(wl)
    assert not g["out"].any() and np.isneginf(g["lse"]).all()
    wl = W.tiny_sol(seed=6, H=1, L=256, d=64)
    wl.lkv_valid = 1
    wl.qk_float = True
    _check_workload(orc, wl)
    wl = W.tiny_sol(seed=6, H=1, L=256, d=64)
    wl.lkv_valid = 1
    wl.rule, wl.sparsity = 1, 0.75
    _check_workload(orc, wl)
    wl = W.tiny_sol(seed=7, H=2, L=512, d=128, valid=300)
    wl.rule, wl.sparsity = 1, 0.99
    g, o = _check_workload(orc, wl)
    assert ((g["map"][..., :5] == 1).sum(-1) == 1).all()


@pytest.mark.parametrize("rule,G", [(0, 1), (1, 0)])
def test_max_key_blocks(sa, orc, rule, G):
    """The longest rows the routing rules accept: 6144 key blocks of 64 rows
    (393216 keys; the forward walks its block map in 12 windows of 512), with
    a ragged end of the keys and of the queries."""
    rng = np.random.default_rng(171 + 64 + rule)
    H, Lq, Lkv, d = 2, 128, 6144 * 64, 64
    lq_valid, lkv_valid = Lq - 3, Lkv - 21
    q = W.iid_normal_bf16(rng, (1, H, Lq, d))
    k = W.iid_normal_bf16(rng, (1, H, Lkv, d))
    v = W.iid_normal_bf16(rng, (1, H, Lkv, d))
    for t in (k, v):
        t[0, :, lkv_valid:] = 0            # padding rows hold zeros
    q[0, :, lq_valid:] = 0
    wl = W.Workload("max_key_blocks", 1, H, Lq, Lkv, d, lq_valid, lkv_valid, q, k, v, threshold=1.0,
                    centroids_per_block=G, kblock=64, k_scale_rows=64)
    wl.rule, wl.sparsity = rule, 0.6
    g, o = _check_workload(orc, wl)
    assert (g["map"] == EXACT).sum() > 4000 and (g["map"] != EXACT).sum() > 1000


@pytest.mark.parametrize("rule,d,G,prefix", [(0, 128, 1, 0), (1, 128, 1, 1024), (0, 64, 2, 1024), (1, 64, 0, 0)])
def test_long_rows(sa, orc, rule, d, G, prefix):
    """Rows with more than 512 candidate key blocks (here up to 640) take the
    decision kernels that recompute the proxies on every pass instead of
    keeping a row's proxies in LDS: the threshold rule's mean and variance
    over several passes, the fixed-sparsity rule's radix select."""
    rng = np.random.default_rng(91 + d + 10 * rule)
    H, Lq, Lkv = 2, 256, 640 * 64
    lq_valid, lkv_valid = Lq - 5, Lkv - 40
    q = W.iid_normal_bf16(rng, (1, H, Lq, d))
    k = W.iid_normal_bf16(rng, (1, H, Lkv, d))
    v = W.iid_normal_bf16(rng, (1, H, Lkv, d))
    for t in (k, v):
        t[0, :, lkv_valid:] = 0            # padding rows hold zeros
    q[0, :, lq_valid:] = 0
    wl = W.Workload("long_rows", 1, H, Lq, Lkv, d, lq_valid, lkv_valid, q, k, v, threshold=1.0,
                    centroids_per_block=G, prefix_tokens=prefix, kblock=64, k_scale_rows=64)
    wl.rule, wl.sparsity = rule, 0.7
    g, o = _check_workload(orc, wl)
    cand = (Lkv - prefix) // 64
    assert cand > 512
    nvalid = -(-lkv_valid // 64) - prefix // 64
    routed = g["map"][..., prefix // 64:prefix // 64 + nvalid]
    if rule == 1:   # the sparsity crosses the boundary as float32: 0.7f * 640 floors to 447
        keep = nvalid - int(np.floor(float(np.float32(0.7)) * nvalid))
        assert ((routed == EXACT).sum(-1) == keep).all()
    else:
        assert 0 < (routed == CENTROID).sum() < routed.size


@pytest.mark.parametrize("rule,G,prefix", [(0, 1, 0), (0, 2, 128), (1, 1, 0)])
def test_batched(sa, orc, rule, G, prefix):
    """B = 2: every kernel indexes (batch, head) pairs, the pooling kernels
    through a batch grid dimension."""
    rng = np.random.default_rng(95 + rule + 3 * G)
    B, H, L, d, valid = 2, 3, 1024, 128, 1000
    q = W.iid_normal_bf16(rng, (B, H, L, d))
    k = W.iid_normal_bf16(rng, (B, H, L, d))
    v = W.iid_normal_bf16(rng, (B, H, L, d))
    for t in (q, k, v):
        t[:, :, valid:] = 0
    wl = W.Workload("batched", B, H, L, L, d, valid, valid, q, k, v, threshold=0.5, centroids_per_block=G,
                    prefix_tokens=prefix, kblock=64, k_scale_rows=64)
    wl.rule, wl.sparsity = rule, 0.5
    g, o = _check_workload(orc, wl)
    assert g["map"].shape[0] == B and not np.array_equal(g["map"][0], g["map"][1])


@pytest.mark.parametrize("rule,G,d,L", [(0, 1, 64, 512), (1, 2, 128, 512), (1, 1, 64, 2560), (1, 0, 128, 512)])
def test_decisions_in_sixteen_row_workgroups(sa, orc, rule, G, d, L):
    """More 32-query-block decision chunks than compute units (260 heads):
    the fixed-sparsity decisions run in 16-row workgroups, two per CU (the
    threshold rule keeps 32-row ones).  L = 2560 gives 20 query blocks per
    head: a full 16-row chunk and a ragged one."""
    wl = W.tiny_sol(seed=111 + rule + d + G + L, H=260, L=L, d=d, valid=L - 42, centroids_per_block=max(G, 1))
    wl.centroids_per_block = G
    wl.rule, wl.sparsity = rule, 0.6
    nQB = L // 128
    g, o = _check_workload(orc, wl, tau=0.5, sel=np.arange(0, 260 * nQB, 7 * nQB // 4 + 1))
    assert (g["map"] == (CENTROID if G > 0 else DROP)).any()
