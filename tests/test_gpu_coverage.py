"""GPU parity for the INT8-V cache with centroids, padding that holds
non-finite values, guard bands around every output, and the routing
statistics.

FlashVSR Kitchen Sparse Attention, opening section: K/V arrive as an INT8
cache with one scale per 128-row slab; Configure Sol Sparse Attention, "How it
works": skipped blocks still contribute their centroids, here built from that
INT8 V.  Padding rows (past the valid length, or between segments) take no part
in the softmax, whatever they hold.
"""
import numpy as np
import pytest
import torch

import workloads as W
from workloads import CENTROID, DROP, EXACT, bf16_bits
from tests.helpers import MAX_ABS, MEAN_ABS, bf16_dev, compare_maps, gpu_pipeline, say
from tests.test_gpu_parity import _check_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import block_sparse_int8_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.device_check(torch.cuda.current_device())
    return m


# ---------------------------------------------------------------------------
# INT8 V with centroids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,G,kblock,vrows", [(128, 1, 64, 128), (128, 2, 64, 64), (64, 1, 64, 128),
                                              (64, 2, 128, 128), (128, 2, 128, 64)])
def test_int8_v_sol_rule_with_centroids(sa, orc, d, G, kblock, vrows):
    """The Sol rule over an INT8 V cache: V-bar dequantized through the V scales,
    the INT8-V forward with centroid columns (d = 64 and 128)."""
    wl = W.tiny_sol(seed=70 + d + G + kblock, H=2, L=1024, d=d, valid=1000, centroids_per_block=G)
    wl.kblock = wl.k_scale_rows = kblock
    wl.v_int8, wl.v_scale_rows = True, vrows
    g, o = _check_workload(orc, wl, tau=0.5)
    assert (g["map"] == CENTROID).any() and (g["map"] == EXACT).any()


@pytest.mark.parametrize("d,G,kblock,ksr", [(128, 1, 128, 64), (128, 2, 128, 64), (64, 2, 128, 128),
                                            (128, 2, 64, 64), (64, 1, 64, 64)])
def test_int8_v_explicit_centroid_map(sa, orc, d, G, kblock, ksr):
    """Explicit maps with EXACT / CENTROID / DROP entries over an INT8 K/V cache,
    including 128-key blocks whose K carries one scale per 64 rows (a centroid
    group then combines two scale blocks)."""
    L, H = 1024, 2
    wl = W.tiny_sol(seed=80 + d + G, H=H, L=L, d=d, valid=1000, centroids_per_block=G)
    wl.kblock, wl.k_scale_rows, wl.map_kblock = kblock, ksr, kblock
    wl.v_int8, wl.v_scale_rows = True, 128
    rng = np.random.default_rng(81 + kblock)
    wl.explicit_map = rng.choice(np.array([EXACT, CENTROID, DROP], np.uint8), size=(1, H, L // 128, L // kblock),
                                 p=[0.45, 0.45, 0.1])
    g, o = _check_workload(orc, wl)
    assert (g["map"] == CENTROID).sum() > 0


def test_int8_v_virtual_table_with_centroids(sa, orc):
    """INT8 V read through the virtual-KV block table (64-row logical blocks
    from physical blocks) with 2x32 centroids: V-bar and the exact tiles both
    read the remapped rows and their scales."""
    wl = W.config(5, small=True)
    wl.v_int8, wl.v_scale_rows = True, 128
    _check_workload(orc, wl)


# ---------------------------------------------------------------------------
# Padding holding non-finite values
# ---------------------------------------------------------------------------

def _poison(bits, rows, values):
    """Copy of bf16 bits with the given rows (indices along L) cycling through values."""
    out = bits.copy()
    pat = bf16_bits(np.array(values, np.float32))
    for n, r in enumerate(rows):
        out[:, :, r, :] = pat[(n + np.arange(bits.shape[3])) % len(pat)]
    return out


@pytest.mark.parametrize("qk_float", [False, True])
def test_nonfinite_padding_is_ignored(sa, qk_float):
    """V rows past the valid length and inside segment padding, and (floating
    path) Q and K rows past the valid length, filled with NaN and +-Inf: the
    outputs, lse, map and centroids equal those of the zero-padded run bit for
    bit.  (K rows inside the layout's padding stay zero: the quantizer does not
    know the layout, and the header asks for zeros there.)"""
    wl = W.ref2va_segments(H=2, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=2,
                           frame_tokens=320, centroids_per_block=2)
    wl.qk_float = qk_float
    ref = gpu_pipeline(wl)
    pad_rows = []
    segs = wl.segments
    for x in range(len(segs)):
        end = int(segs[x][0] + segs[x][1])
        nxt = int(segs[x + 1][0]) if x + 1 < len(segs) else wl.Lkv
        pad_rows += list(range(end, nxt))
    assert len(pad_rows) > 64
    vals = [np.nan, np.inf, -np.inf, 3.0e38]
    bad = W.Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
    bad.v = _poison(wl.v, pad_rows, vals)
    tail = list(range(wl.lkv_valid, wl.Lkv))
    if qk_float:
        bad.q = _poison(wl.q, list(range(wl.lq_valid, wl.Lq)), vals)
        bad.k = _poison(wl.k, tail, vals)
    say(f"case nonfinite padding qk_float={qk_float}: {len(pad_rows)} V rows, {len(tail)} tail rows")
    got = gpu_pipeline(bad)
    for key in ("map", "kbar", "vbar", "count", "out", "lse"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.isfinite(got["out"]).all()


# ---------------------------------------------------------------------------
# Guard bands around the outputs
# ---------------------------------------------------------------------------

GUARD = 4096
FILL = 0xA5


def _guarded(shape, dtype):
    """A tensor of `shape` inside a byte buffer with GUARD bytes of FILL on each
    side; returns (tensor, buffer)."""
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((nbytes + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
    t = buf[GUARD:GUARD + nbytes].view(dtype).view(shape)
    return t, buf


def _guards_intact(buf):
    h = buf.cpu().numpy()
    return bool((h[:GUARD] == FILL).all() and (h[-GUARD:] == FILL).all())


@pytest.mark.parametrize("case", ["tiny_sol", "segments_2x32", "segments_topk", "float_qk"])
def test_guard_bands_untouched(sa, orc, case):
    """Quantized Q/K, scales, map, centroids, counts, row statistics, output
    and lse are written into buffers with guard bands of a known byte on both
    sides; after quantize, route and forward the guards are unchanged and the
    results still match the oracle."""
    if case == "tiny_sol":
        wl = W.config(1)
    else:
        wl = W.ref2va_segments(H=2, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=2,
                               frame_tokens=320, centroids_per_block=2)
        if case == "segments_topk":
            wl.rule, wl.sparsity = 1, 0.75
        if case == "float_qk":
            wl.qk_float = True
    say(f"case guards {case}")
    B, H, Lq, d = wl.q.shape
    Lkv, G, kb = wl.Lkv, wl.centroids_per_block, wl.kblock
    nQB, nKB = Lq // 128, Lkv // kb
    bufs = []

    def g(shape, dtype):
        t, b = _guarded(shape, dtype)
        bufs.append(b)
        return t

    q, k, v = bf16_dev(wl.q), bf16_dev(wl.k), bf16_dev(wl.v)
    q8, qs = sa.quantize_qk_int8(q, wl.lq_valid, 128, out=g((B, H, Lq, d), torch.int8),
                                 scale=g((B, H, nQB), torch.float32))
    k8, ks = sa.quantize_qk_int8(k, wl.lkv_valid, kb, out=g((B, H, Lkv, d), torch.int8),
                                 scale=g((B, H, Lkv // kb), torch.float32))
    outs = dict(map=g((B, H, nQB, nKB), torch.uint8), k_centroid=g((B, H, nKB, G, d), torch.float32),
                v_centroid=g((B, H, nKB, G, d), torch.float32), count=g((B, H, nKB, G), torch.float32),
                row_stats=g((B, H, nQB, 2), torch.float64))
    r = sa.sparse_attn_route(q8, k8, ks, v, lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid, threshold=wl.threshold,
                             centroids_per_block=G, kblock=kb, rule=wl.rule, sparsity=wl.sparsity,
                             segments=wl.segments, outputs=outs, row_stats=True)
    out, lse = g((B, H, Lq, d), torch.float32), g((B, H, Lq), torch.float32)
    kw = dict(k_centroid=r["k_centroid"], v_centroid=r["v_centroid"], count=r["count"], lq_valid=wl.lq_valid,
              lkv_valid=wl.lkv_valid, centroids_per_block=G, kblock=kb, sm_scale=wl.sm_scale, out=out, lse=lse,
              return_lse=True, segments=wl.segments)
    if wl.qk_float:
        sa.sparse_attn_fwd_float(q, k, v, r["map"], **kw)
    else:
        sa.sparse_attn_fwd(q8, qs, k8, ks, v, r["map"], **kw)
    torch.cuda.synchronize()
    for n, b in enumerate(bufs):
        assert _guards_intact(b), f"guard band of buffer {n} was written"
    assert r["row_stats"].data_ptr() == outs["row_stats"].data_ptr()
    o = orc.run(wl)
    bad, _, _ = compare_maps(r["map"].cpu().numpy(), o["map"], o["tie"])
    assert bad == 0
    diff = np.abs(out.cpu().numpy().reshape(B * H, Lq, d) - o["out"].reshape(B * H, Lq, d))[:, :wl.lq_valid]
    assert diff.max() <= MAX_ABS and diff.mean() <= MEAN_ABS


# ---------------------------------------------------------------------------
# Routing statistics and proxies at partial blocks
# ---------------------------------------------------------------------------

def test_row_stats_and_partial_block_proxies(sa, orc):
    """The threshold rule's per-row mean and population std against the
    oracle's float64 values (the only difference is the summation order, a few
    ulps), on a layout with partial key blocks at every segment end; and the
    fixed-sparsity rule on the same layout bit-exact with no tie band, which
    holds only if the proxies of partial blocks (n < 64) are the oracle's
    float64 values bit for bit."""
    wl = W.ref2va_segments(H=3, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=3,
                           frame_tokens=333, centroids_per_block=1)
    ends = [int(s[0] + s[1]) for s in wl.segments]
    assert any(e % 64 for e in ends)
    g = gpu_pipeline(wl)
    o = orc.run(wl)
    st = np.isfinite(o["stats"])
    assert st.all()
    # mu and sigma of a row within 1e-12 of |mu| + sigma (the tie band is 1e-6 sigma)
    mu, sig = o["stats"][..., 0], o["stats"][..., 1]
    scale = (np.abs(mu) + sig)[..., None]
    err = np.abs(g["stats"] - o["stats"]) / scale
    assert err.max() < 1e-12, err.max()
    for sp in (0.3, 0.5, 0.75, 0.9):
        wl.rule, wl.sparsity = 1, sp
        g = gpu_pipeline(wl)
        o = orc.run(wl)
        assert np.array_equal(g["map"], o["map"]), sp


# ---------------------------------------------------------------------------
# Column sums from the quantizer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,R,SR,L,valid", [(128, 64, 32, 1024, 1000), (128, 64, 64, 1024, 1000),
                                            (128, 128, 128, 1024, 1000), (128, 128, 32, 1024, 1000),
                                            (64, 64, 32, 512, 300), (64, 128, 128, 512, 512),
                                            (64, 128, 32, 512, 77), (128, 128, 128, 256, 0)])
def test_quantize_column_sums(sa, orc, d, R, SR, L, valid):
    """The quantizer's optional column sums equal the sums of the oracle's codes
    over every chunk of SR rows (padding rows coded 0), and the codes are the
    same whether or not the sums are written."""
    say(f"case col sums d={d} R={R} SR={SR} L={L} valid={valid}")
    rng = np.random.default_rng(d + R + L + valid + SR)
    x = rng.standard_normal((2, 3, L, d), dtype=np.float32) * rng.uniform(0.1, 10, (2, 3, 1, 1)).astype(np.float32)
    if L >= 2 * R:
        # a block of codes +-127 with one sign per column: sums reach +-127 * SR
        x[1, 1, :R] = np.float32(127.0 / 64) * np.sign(rng.standard_normal(d)).astype(np.float32)[None, :]
    xb = bf16_bits(x)
    g8, gs, gsum = sa.quantize_qk_int8(bf16_dev(xb), valid, R, col_sums=True, sum_rows=SR)
    o8, os_ = orc.quantize(xb, valid, R)
    assert np.array_equal(g8.cpu().numpy(), o8) and np.array_equal(gs.cpu().numpy(), os_)
    ref = o8.astype(np.int64).reshape(2, 3, L // SR, SR, d).sum(axis=3)
    assert gsum.dtype == torch.int16 and np.array_equal(gsum.cpu().numpy().astype(np.int64), ref)
    # a strided view ([B,L,H,d] memory)
    blhd = bf16_dev(np.ascontiguousarray(xb.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)
    _, _, gsum2 = sa.quantize_qk_int8(blhd, valid, R, col_sums=True, sum_rows=SR)
    assert np.array_equal(gsum2.cpu().numpy(), gsum.cpu().numpy())


def _sums_cases():
    c3 = W.config(3, small=True)
    c4 = W.config(4, small=True)
    k128 = W.tiny_sol(seed=90, H=2, L=1024, d=128, valid=1000, centroids_per_block=2)
    k128.kblock = k128.k_scale_rows = 128
    topk = W.config(3, small=True)
    topk.rule, topk.sparsity = 1, 0.75
    seg = W.ref2va_segments(H=2, text=77, ref_image=300, ref_audio=40, ref_video_frames=1, video_frames=2,
                            frame_tokens=320, centroids_per_block=2)
    cache = W.tiny_sol(seed=91, H=2, L=1024, d=128, valid=1000, centroids_per_block=2)
    cache.kblock, cache.k_scale_rows, cache.map_kblock = 128, 64, 128
    cache.v_int8, cache.v_scale_rows = True, 128
    cache.explicit_map = np.random.default_rng(92).choice(np.array([EXACT, CENTROID, DROP], np.uint8),
                                                          size=(1, 2, 8, 8), p=[0.45, 0.45, 0.1])
    d64 = W.tiny_sol(seed=93, H=3, L=640, d=64, valid=577, centroids_per_block=1)
    return {"tiny": W.config(1), "wan_small": c3, "prefix_2x32": c4, "kblock128": k128, "topk": topk,
            "segments": seg, "int8_cache_explicit": cache, "d64": d64}


@pytest.mark.parametrize("name", list(_sums_cases().keys()))
def test_route_from_sums_equals_route_from_codes(sa, name):
    """The route fed the quantizer's column sums gives the same map, centroids,
    counts and statistics, and the forward the same output, as the route that
    sums the codes itself, bit for bit."""
    wl = _sums_cases()[name]
    say(f"case sums vs codes {name}")
    a = gpu_pipeline(wl, sums=True)
    b = gpu_pipeline(wl, sums=False)
    assert a["k_sums"] is not None
    for key in ("map", "kbar", "vbar", "count", "stats", "out", "lse"):
        if a[key] is None:
            continue
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_route_reads_no_codes_when_given_sums(sa):
    """Through the C ABI: with q_sums and k_sums the route accepts NULL q and k
    and gives the binding's result."""
    import ctypes
    wl = W.config(3, small=True)
    q8, qs, qsum = sa.quantize_qk_int8(bf16_dev(wl.q), wl.lq_valid, 128, col_sums=True, sum_rows=128)
    k8, ks, ksum = sa.quantize_qk_int8(bf16_dev(wl.k), wl.lkv_valid, 64, col_sums=True, sum_rows=32)
    v = bf16_dev(wl.v)
    ref = sa.sparse_attn_route(q8, k8, ks, v, lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid, threshold=1.0,
                               centroids_per_block=1, row_stats=True)
    B, H, Lq, d = q8.shape
    nQB, nKB = Lq // 128, wl.Lkv // 64
    dims = sa.sa_dims(B, H, Lq, wl.Lkv, d, wl.lq_valid, wl.lkv_valid, wl.Lkv)
    prm = sa._params(1.0, 1, 0, 64, 64, 128, 64)
    lib = sa.load()
    ws_bytes = lib.sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    bmap = torch.empty((B, H, nQB, nKB), dtype=torch.uint8, device="cuda")
    kc = torch.empty((B, H, nKB, 1, d), dtype=torch.float32, device="cuda")
    vc, cnt = torch.empty_like(kc), torch.empty((B, H, nKB, 1), dtype=torch.float32, device="cuda")
    st = torch.empty((B, H, nQB, 2), dtype=torch.float64, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.sparse_attn_route(None, None, P(ks), P(v), sa.SA_BF16, None, None, P(qsum), P(ksum), ctypes.byref(dims),
                               ctypes.byref(prm), None, P(bmap), P(kc), P(vc), P(cnt), P(st), P(ws), ws_bytes,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.sa_last_error()
    torch.cuda.synchronize()
    for got, key in ((bmap, "map"), (kc, "k_centroid"), (vc, "v_centroid"), (cnt, "count"), (st, "row_stats")):
        assert torch.equal(got, ref[key]), key


# ---------------------------------------------------------------------------
# Neighbouring query blocks with different maps (d = 128, bf16 V)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,L,valid", [(1, 1152, 1100), (2, 1024, 1000), (0, 640, 577)])
def test_neighbouring_blocks_with_differing_maps(sa, orc, G, L, valid):
    """Neighbouring query blocks keep different tiles (random explicit maps),
    with an odd number of query blocks and tiles that hold the end of the
    valid keys."""
    H = 3
    wl = W.tiny_sol(seed=140 + G + L, H=H, L=L, d=128, valid=valid, centroids_per_block=max(G, 1))
    wl.centroids_per_block = G
    rng = np.random.default_rng(141 + G)
    states = np.array([EXACT, CENTROID, DROP] if G > 0 else [EXACT, DROP], np.uint8)
    probs = [0.5, 0.35, 0.15] if G > 0 else [0.6, 0.4]
    wl.explicit_map = rng.choice(states, size=(1, H, L // 128, L // 64), p=probs)
    g, o = _check_workload(orc, wl)
    gm = g["map"]
    assert (gm[:, :, 0::2][:, :, :gm.shape[2] // 2] != gm[:, :, 1::2]).any()


def test_dropped_tile_does_not_reach_a_block(sa, orc):
    """A tile that one query block keeps and its neighbour drops reaches only
    the block that keeps it: a NaN or Inf in its V rows leaves the other
    block's outputs as they are without the tile."""
    H, L = 1, 512
    wl = W.tiny_sol(seed=150, H=H, L=L, d=128, valid=L, centroids_per_block=1)
    wl.centroids_per_block = 0
    em = np.full((1, H, L // 128, L // 64), EXACT, np.uint8)
    em[0, 0, 0::2, 3] = DROP       # blocks 0 and 2 drop key blocks 3 and 5, blocks 1 and 3 keep them
    em[0, 0, 0::2, 5] = DROP
    wl.explicit_map = em
    v = wl.v.copy()
    v[0, 0, 3 * 64 + 7, 11] = 0x7FC0     # bf16 NaN in a valid row of key block 3
    v[0, 0, 5 * 64 + 60, 0] = 0x7F80     # bf16 +Inf in key block 5
    wl.v = v
    say("case non-finite V in tiles that every other query block drops")
    g = gpu_pipeline(wl)
    o = orc.run(wl)
    out = g["out"].reshape(4, 128, 128)
    assert np.isfinite(out[0]).all() and np.isfinite(out[2]).all()
    assert not np.isfinite(out[1]).all() and not np.isfinite(out[3]).all()
    for b in (0, 2):
        err = np.abs(out[b] - o["out"][b])
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
