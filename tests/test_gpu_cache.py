"""GPU parity of the streaming INT8 K/V cache (FlashVSR Kitchen Sparse
Attention, opening section: a sliding INT8 cache of past K/V in bounded
128-row slabs) and of attention read straight from the ring."""
import numpy as np
import pytest
import torch

from workloads import bf16_bits, EXACT
from tests.helpers import MAX_ABS, MEAN_ABS, bf16_dev, compare_outputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import block_sparse_int8_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.device_check(torch.cuda.current_device())
    return m


def _stream(seed, H, rows, d, B=1):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((B, H, rows, d)).astype(np.float32))


@pytest.mark.parametrize("d,R,B", [(128, 128, 1), (64, 64, 1), (128, 128, 2)])
def test_cache_appends_bitexact(sa, orc, d, R, B):
    """Chunks with wrap-around and a partial last slab, against the oracle's
    ring after the same appends."""
    H, slots = 3, 6
    chunks = [(3, None), (2, None), (4, None), (2, R + 40)]   # (slabs, valid rows)
    total = sum(n for n, _ in chunks)
    x = _stream(41, H, total * R, d, B)
    gq = torch.zeros((B, H, slots * R, d), dtype=torch.int8, device="cuda")
    gs = torch.zeros((B, H, slots), dtype=torch.float32, device="cuda")
    oq = np.zeros((B, H, slots * R, d), np.int8)
    osc = np.zeros((B, H, slots), np.float32)
    g = 0
    slot = 0
    for n, valid in chunks:
        part = x[:, :, g * R:(g + n) * R]
        say(f"case cache append B={B} d={d} R={R} slabs={n} first_slot={slot} valid={valid}")
        nxt = sa.kv_cache_append_int8(bf16_dev(part), gq, gs, slot, valid_len=valid, rows_per_slab=R)
        orc.cache_append(oq, osc, part, first_slot=slot, valid_len=valid, rows_per_slab=R)
        assert nxt == (slot + n) % slots
        slot = nxt
        g += n
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), oq)
    assert np.array_equal(gs.cpu().numpy(), osc)


def test_cache_append_strided_chunk(sa, orc):
    """A chunk that is a strided view (rows of a larger [B,H,L,d] buffer)."""
    H, d, R, slots = 2, 128, 128, 4
    x = _stream(42, H, 8 * R, d)
    xv = bf16_dev(x)[:, :, 2 * R:5 * R]          # non-contiguous over H
    gq = torch.zeros((1, H, slots * R, d), dtype=torch.int8, device="cuda")
    gs = torch.zeros((1, H, slots), dtype=torch.float32, device="cuda")
    sa.kv_cache_append_int8(xv, gq, gs, 2, rows_per_slab=R)
    oq = np.zeros((1, H, slots * R, d), np.int8)
    osc = np.zeros((1, H, slots), np.float32)
    orc.cache_append(oq, osc, x[:, :, 2 * R:5 * R], first_slot=2, rows_per_slab=R)
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), oq) and np.array_equal(gs.cpu().numpy(), osc)


def test_attention_over_the_ring(sa, orc):
    """Five frames of 512 tokens streamed into rings of 12 slabs (three frames)
    for K and V.  The current frame's queries attend the cached frames under a
    local-causal map (frames t-1..t, in-frame block within +-2) given in slot
    order; the oracle attends the same frames in time order with the map in
    time order.  Attention is order-free over keys, so the outputs agree."""
    H, d, R, F, T = 2, 128, 128, 512, 5
    slots = 3 * F // R
    bpf = F // R
    rng = np.random.default_rng(43)
    q_all = bf16_bits(rng.standard_normal((1, H, T * F, d)).astype(np.float32))
    k_all = bf16_bits(rng.standard_normal((1, H, T * F, d)).astype(np.float32))
    v_all = bf16_bits(rng.standard_normal((1, H, T * F, d)).astype(np.float32))
    kq = torch.zeros((1, H, slots * R, d), dtype=torch.int8, device="cuda")
    ks = torch.zeros((1, H, slots), dtype=torch.float32, device="cuda")
    vq = torch.zeros_like(kq)
    vs = torch.zeros_like(ks)
    slot = 0
    for t in range(T):
        fr = slice(t * F, (t + 1) * F)
        sa.kv_cache_append_int8(bf16_dev(k_all[:, :, fr]), kq, ks, slot, rows_per_slab=R)
        slot = sa.kv_cache_append_int8(bf16_dev(v_all[:, :, fr]), vq, vs, slot, rows_per_slab=R)
    # cached frames T-3..T-1 in time order; slot of the g-th global slab is g % slots
    g0 = (T - 3) * bpf
    slot_of_logical = np.array([(g0 + j) % slots for j in range(slots)])
    # queries: the last frame; map over the three cached frames in time order
    nq = bpf
    lmap = np.zeros((1, H, nq, slots), np.uint8)
    for qi in range(nq):
        for kj in range(slots):
            tf, b2 = divmod(kj, bpf)
            if tf in (1, 2) and abs(b2 - qi) <= 2:   # frames T-2, T-1 relative to the cache start
                lmap[..., qi, kj] = EXACT
    smap = np.zeros_like(lmap)
    smap[..., slot_of_logical] = lmap
    q = bf16_dev(q_all[:, :, (T - 1) * F:T * F])
    q8, qsc = sa.quantize_qk_int8(q, F, 128)
    r = sa.sparse_attn_route(q8, kq, ks, vq, v_scale=vs, centroids_per_block=0, kblock=128, k_scale_rows=128,
                             v_scale_rows=128, explicit_map=torch.from_numpy(smap).cuda(), map_kblock=128)
    out = sa.sparse_attn_fwd(q8, qsc, kq, ks, vq, r["map"], v_scale=vs, centroids_per_block=0, kblock=128,
                             k_scale_rows=128, v_scale_rows=128)
    torch.cuda.synchronize()
    assert np.array_equal(r["map"].cpu().numpy(), smap)
    # oracle in time order
    kq_h, ks_h, vq_h, vs_h = kq.cpu().numpy(), ks.cpu().numpy(), vq.cpu().numpy(), vs.cpu().numpy()
    idx = np.concatenate([np.arange(s * R, (s + 1) * R) for s in slot_of_logical])
    k_log, v_log = kq_h[:, :, idx], vq_h[:, :, idx]
    ks_log, vs_log = ks_h[:, :, slot_of_logical], vs_h[:, :, slot_of_logical]
    # the ring holds exactly the last three frames, quantized per slab
    kq_ref, ks_ref = orc.quantize(k_all[:, :, (T - 3) * F:], rows_per_block=R)
    assert np.array_equal(k_log, kq_ref) and np.array_equal(ks_log, ks_ref)
    o8, osc = orc.quantize(q_all[:, :, (T - 1) * F:T * F], rows_per_block=128)
    ro = orc.route(o8, k_log, ks_log, 128, F, slots * R, v8=v_log, v_scale=vs_log, v_scale_rows=128, G=0,
                   kblock=128, explicit_map=lmap, map_kblock=128)
    oo, lse, sel = orc.forward(o8, osc, k_log, ks_log, 128, F, slots * R, ro["map"], v8=v_log, v_scale=vs_log,
                               v_scale_rows=128, kblock=128, G=0)
    mx, mean, rows = compare_outputs(out.cpu().numpy(), oo, sel, nq, F, F)
    say(f"  ring attention: rows {rows}, max-abs {mx:.3e}, mean-abs {mean:.3e}")
    assert rows == H * F and mx <= MAX_ABS and mean <= MEAN_ABS
