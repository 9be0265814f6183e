"""Pins for the oracle's streaming INT8 K/V cache (CPU only).

FlashVSR Kitchen Sparse Attention, opening section: in streaming use each
block holds the recent K/V history as INT8, bounded, in 128-row slabs.  The
cache is a ring of slabs; each new slab evicts the oldest.
"""
import numpy as np
import pytest

from workloads import bf16_bits


def _stream(seed, H, n_slabs, d=128, R=128):
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((1, H, n_slabs * R, d)).astype(np.float32))


@pytest.mark.parametrize("chunks", [[3, 2, 4, 1], [6, 6], [1] * 9, [5, 4]])
def test_chunked_appends_equal_one_quantization_of_the_stream(orc, chunks):
    """Whatever the chunking, the ring holds the last `slots` slabs of the
    stream, slab g in slot g mod slots, bit for bit as one quantization of the
    whole stream gives them."""
    H, d, R, slots = 2, 128, 128, 6
    total = sum(chunks)
    x = _stream(7, H, total, d, R)
    cq = np.zeros((1, H, slots * R, d), np.int8)
    cs = np.zeros((1, H, slots), np.float32)
    g = 0
    for n in chunks:
        orc.cache_append(cq, cs, x[:, :, g * R:(g + n) * R], first_slot=g % slots, rows_per_slab=R)
        g += n
    q_all, s_all = orc.quantize(x, rows_per_block=R)
    for gs in range(max(0, total - slots), total):
        slot = gs % slots
        assert np.array_equal(cq[0, :, slot * R:(slot + 1) * R], q_all[0, :, gs * R:(gs + 1) * R])
        assert np.array_equal(cs[0, :, slot], s_all[0, :, gs])
    if total < slots:   # never-written slots keep their contents
        assert (cq[0, :, total * R:] == 0).all() and (cs[0, :, total:] == 0).all()


def test_partial_last_slab_codes_padding_zero(orc):
    H, d, R, slots = 1, 64, 128, 4
    x = _stream(8, H, 2, d, R)
    cq = np.full((1, H, slots * R, d), 5, np.int8)
    cs = np.full((1, H, slots), 9.0, np.float32)
    orc.cache_append(cq, cs, x, first_slot=3, valid_len=200, rows_per_slab=R)
    q_ref, s_ref = orc.quantize(x, valid_len=200, rows_per_block=R)
    assert np.array_equal(cq[0, :, 3 * R:4 * R], q_ref[0, :, :R])      # slab 0 -> slot 3
    assert np.array_equal(cq[0, :, 0:R], q_ref[0, :, R:])              # slab 1 wraps to slot 0
    assert (cq[0, :, 0 + 72:R] == 0).all()                             # rows 200.. of the chunk: padding
    assert (cq[0, :, R:3 * R] == 5).all() and (cs[0, :, 1:3] == 9.0).all()   # untouched slots


def test_rejects_overfull_chunk(orc):
    x = _stream(9, 1, 5, 64, 128)
    cq = np.zeros((1, 1, 4 * 128, 64), np.int8)
    cs = np.zeros((1, 1, 4), np.float32)
    with pytest.raises(ValueError):
        orc.cache_append(cq, cs, x, first_slot=0)


def test_attention_over_ring_in_slot_order_equals_time_order(orc):
    """Keys in ring (slot) order with the map permuted the same way give the
    attention of the time-ordered keys: the softmax is order-free over keys."""
    from workloads import EXACT
    H, d, R, F, T = 1, 64, 128, 256, 4
    slots, bpf = 2 * F // R, F // R
    rng = np.random.default_rng(44)
    q_all, k_all, v_all = (bf16_bits(rng.standard_normal((1, H, T * F, d)).astype(np.float32)) for _ in range(3))
    kq = np.zeros((1, H, slots * R, d), np.int8)
    ks = np.zeros((1, H, slots), np.float32)
    vq, vs = kq.copy(), ks.copy()
    slot = 0
    for t in range(T):
        fr = slice(t * F, (t + 1) * F)
        orc.cache_append(kq, ks, k_all[:, :, fr], slot)
        orc.cache_append(vq, vs, v_all[:, :, fr], slot)
        slot = (slot + bpf) % slots
    order = np.array([((T - 2) * bpf + j) % slots for j in range(slots)])   # slot of each time-ordered slab
    lmap = np.full((1, H, bpf, slots), EXACT, np.uint8)
    lmap[..., 0] = 0
    smap = np.zeros_like(lmap)
    smap[..., order] = lmap
    o8, osc = orc.quantize(q_all[:, :, (T - 1) * F:], rows_per_block=128)
    idx = np.concatenate([np.arange(s * R, (s + 1) * R) for s in order])
    a = orc.forward(o8, osc, kq[:, :, idx], ks[:, :, order], 128, F, slots * R, lmap, v8=vq[:, :, idx],
                    v_scale=vs[:, :, order], v_scale_rows=128, kblock=128, G=0)[0]
    b = orc.forward(o8, osc, kq, ks, 128, F, slots * R, smap, v8=vq, v_scale=vs, v_scale_rows=128, kblock=128,
                    G=0)[0]
    assert np.abs(a - b).max() < 1e-12
    # and the ring holds the last two frames, quantized per slab
    kq_ref, _ = orc.quantize(k_all[:, :, (T - 2) * F:], rows_per_block=R)
    assert np.array_equal(kq[:, :, idx], kq_ref)
