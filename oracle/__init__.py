"""CPU oracle for block-sparse INT8 video attention (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU path in
``block_sparse_int8_amd`` never imports it, and it imports nothing from there;
the two share only the seeded input generators in ``workloads``.

The arithmetic lives in ``oracle.c`` (plain C, float64 softmax, exact-integer
routing proxies); this module only checks shapes and passes numpy buffers.
Each function names the passage of the pages it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DROP, EXACT, CENTROID = 0, 1, 2
QBLOCK = 128


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        _LIB = ctypes.CDLL(path)
        _LIB.orc_num_threads.restype = ctypes.c_int
        _LIB.orc_route.restype = ctypes.c_int
        _LIB.orc_cache_append.restype = ctypes.c_int
    return _LIB


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_lib().orc_num_threads())


def quantize(x_bits: np.ndarray, valid_len: Optional[int] = None, rows_per_block: int = 128):
    """Per-block symmetric INT8 quantization of a bf16 [B,H,L,d] tensor.
    Returns (codes int8 [B,H,L,d], scales float32 [B,H,ceil(L/R)])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    B, H, L, d = x.shape
    valid_len = L if valid_len is None else valid_len
    nblk = -(-L // rows_per_block)
    q = np.empty((B, H, L, d), dtype=np.int8)
    s = np.empty((B, H, nblk), dtype=np.float32)
    _lib().orc_quantize(_p(x), ctypes.c_int64(H * L * d), ctypes.c_int64(L * d), ctypes.c_int64(d),
                        B, H, L, d, valid_len, rows_per_block, _p(q), _p(s))
    return q, s


def cache_append(cache_q: np.ndarray, cache_scale: np.ndarray, x_bits: np.ndarray, first_slot: int,
                 valid_len: Optional[int] = None, rows_per_slab: int = 128):
    """Streaming INT8 cache: quantize the bf16 chunk [B,H,rows,d] per slab and
    write slab s into ring slot (first_slot + s) % slots of ``cache_q``
    [B,H,slots*R,d] / ``cache_scale`` [B,H,slots] (updated in place)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    B, H, rows, d = x.shape
    slots = cache_scale.shape[2]
    assert cache_q.flags.c_contiguous and cache_scale.flags.c_contiguous
    assert cache_q.dtype == np.int8 and cache_scale.dtype == np.float32
    valid_len = rows if valid_len is None else valid_len
    rc = _lib().orc_cache_append(_p(x), ctypes.c_int64(H * rows * d), ctypes.c_int64(rows * d), ctypes.c_int64(d),
                                 B, H, rows, d, valid_len, rows_per_slab, _p(cache_q), _p(cache_scale), slots,
                                 first_slot)
    if rc != 0:
        raise ValueError("oracle cache_append rejected its arguments")
    return cache_q, cache_scale


def _segments(segments):
    if segments is None or len(segments) == 0:
        return None
    return np.ascontiguousarray(np.asarray(segments, dtype=np.int32).reshape(-1, 3))


def route(q8, k8, k_scale, k_scale_rows, lq_valid, lkv_valid, *, v_bits=None, v8=None, v_scale=None,
          v_scale_rows=128, v_block_src=None, tau=1.0, G=1, prefix=0, kblock=64,
          explicit_map=None, map_kblock=None, rule=0, sparsity=0.0, segments=None):
    """Block map, centroids and routing statistics for one attention call.
    ``rule`` 0 is the threshold rule (``tau``), 1 the fixed-sparsity rule
    (``sparsity``, taken at float32 precision as the library's parameter is).
    ``segments`` (int [n, 3]: start, rows, routed) describes the key layout in
    place of ``prefix``.
    Returns a dict with map uint8 [B,H,nQB,nKB], kbar/vbar float64
    [B,H,nKB,G,d], count float64 [B,H,nKB,G], stats float64 [B,H,nQB,2]
    (mu, sigma; NaN for explicit maps and the fixed-sparsity rule) and tie
    uint8 [B,H,nQB,nKB]."""
    q8 = np.ascontiguousarray(q8, dtype=np.int8)
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    vb = None if v_bits is None else np.ascontiguousarray(v_bits, dtype=np.uint16)
    vi = None if v8 is None else np.ascontiguousarray(v8, dtype=np.int8)
    vsrc = vb if vb is not None else vi
    if vsrc is None:
        raise ValueError("V is required")
    Lv = vsrc.shape[2]
    vsc = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    vbs = None if v_block_src is None else np.ascontiguousarray(v_block_src, dtype=np.int32)
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    nQB = -(-Lq // QBLOCK)
    nKB = -(-Lkv // kblock)
    Gs = max(G, 1)
    out_map = np.zeros((B, H, nQB, nKB), dtype=np.uint8)
    tie = np.zeros((B, H, nQB, nKB), dtype=np.uint8)
    kbar = np.zeros((B, H, nKB, Gs, d), dtype=np.float64)
    vbar = np.zeros((B, H, nKB, Gs, d), dtype=np.float64)
    count = np.zeros((B, H, nKB, Gs), dtype=np.float64)
    stats = np.zeros((B, H, nQB, 2), dtype=np.float64)
    em = None
    if explicit_map is not None:
        em = np.ascontiguousarray(explicit_map, dtype=np.uint8)
        if map_kblock is None:
            map_kblock = kblock
        if em.shape != (B, H, nQB, -(-Lkv // map_kblock)):
            raise ValueError(f"explicit map shape {em.shape}")
    sg = _segments(segments)
    rc = _lib().orc_route(_p(q8), _p(k8), _p(ks), k_scale_rows, _p(vb), _p(vi), _p(vsc), v_scale_rows,
                          _p(vbs), Lv, B, H, Lq, Lkv, d, lq_valid, lkv_valid, int(rule), ctypes.c_double(tau),
                          ctypes.c_double(float(np.float32(sparsity))), G,
                          prefix, kblock, _p(sg), 0 if sg is None else len(sg), _p(em), map_kblock or kblock,
                          _p(out_map), _p(kbar), _p(vbar),
                          _p(count), _p(stats), _p(tie))
    if rc != 0:
        raise ValueError("oracle route rejected its arguments")
    return dict(map=out_map, kbar=kbar, vbar=vbar, count=count, stats=stats, tie=tie)


def forward(q8, q_scale, k8, k_scale, k_scale_rows, lq_valid, lkv_valid, block_map, *, kbar=None,
            vbar=None, count=None, v_bits=None, v8=None, v_scale=None, v_scale_rows=128,
            v_block_src=None, kblock=64, G=1, sm_scale=None, sel: Optional[Sequence[int]] = None,
            segments=None, q_bits=None, k_bits=None):
    """Attention output for the selected query blocks (all when ``sel`` is None).
    With ``q_bits``/``k_bits`` (bf16 [B,H,L,d]) the exact logits and the
    centroid logits use the bf16 Q/K (the floating QK path).
    ``sel`` entries are (b*H + h)*nQB + i.  Returns (out float64 [nsel,128,d],
    lse float64 [nsel,128], sel)."""
    q8 = np.ascontiguousarray(q8, dtype=np.int8)
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    nQB = -(-Lq // QBLOCK)
    vb = None if v_bits is None else np.ascontiguousarray(v_bits, dtype=np.uint16)
    vi = None if v8 is None else np.ascontiguousarray(v8, dtype=np.int8)
    Lv = (vb if vb is not None else vi).shape[2]
    vsc = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    vbs = None if v_block_src is None else np.ascontiguousarray(v_block_src, dtype=np.int32)
    if sel is None:
        sel = np.arange(B * H * nQB, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    out = np.zeros((len(sel), QBLOCK, d), dtype=np.float64)
    lse = np.zeros((len(sel), QBLOCK), dtype=np.float64)
    Gs = max(G, 1)
    nKB = -(-Lkv // kblock)
    if kbar is None:
        kbar = np.zeros((B, H, nKB, Gs, d))
        vbar = np.zeros((B, H, nKB, Gs, d))
        count = np.zeros((B, H, nKB, Gs))
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    sg = _segments(segments)
    _lib().orc_forward(_p(q8), _p(np.ascontiguousarray(q_scale, dtype=np.float32)), _p(k8),
                       _p(np.ascontiguousarray(k_scale, dtype=np.float32)), k_scale_rows, _p(vb), _p(vi),
                       _p(vsc), v_scale_rows, _p(vbs), Lv, B, H, Lq, Lkv, d, lq_valid, lkv_valid, kblock,
                       _p(sg), 0 if sg is None else len(sg), G,
                       _p(np.ascontiguousarray(block_map, dtype=np.uint8)),
                       _p(np.ascontiguousarray(kbar, dtype=np.float64)),
                       _p(np.ascontiguousarray(vbar, dtype=np.float64)),
                       _p(np.ascontiguousarray(count, dtype=np.float64)), ctypes.c_double(sm),
                       _p(sel), len(sel), _p(out), _p(lse),
                       _p(None if q_bits is None else np.ascontiguousarray(q_bits, dtype=np.uint16)),
                       _p(None if k_bits is None else np.ascontiguousarray(k_bits, dtype=np.uint16)))
    return out, lse, sel


def materialize_virtual_k(k_phys_bits, rows_per_slice, src, cos, sin, rot_offset=0):
    """Conservative virtual K: bf16 [B,H,n_logical*S,d]."""
    kp = np.ascontiguousarray(k_phys_bits, dtype=np.uint16)
    B, H, Lp, d = kp.shape
    S = rows_per_slice
    src = np.ascontiguousarray(src, dtype=np.int32)
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    nl = len(src)
    out = np.empty((B, H, nl * S, d), dtype=np.uint16)
    _lib().orc_materialize_virtual_k(_p(kp), B, H, S, Lp // S, d, _p(src), nl, _p(cos), _p(sin),
                                     rot_offset, 2 * cos.shape[1], _p(out))
    return out


def gather_virtual_kv(k_phys_bits, rows_per_slice, src, cos, sin, rot_offset=0, rows_per_block=64):
    """Fast virtual K: INT8 logical keys, scales per 64 logical rows, and the V
    block source table.  Returns (k8, k_scale, v_block_src)."""
    kp = np.ascontiguousarray(k_phys_bits, dtype=np.uint16)
    B, H, Lp, d = kp.shape
    S = rows_per_slice
    src = np.ascontiguousarray(src, dtype=np.int32)
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    nl = len(src)
    Ll = nl * S
    k8 = np.empty((B, H, Ll, d), dtype=np.int8)
    ks = np.empty((B, H, -(-Ll // rows_per_block)), dtype=np.float32)
    vbs = np.empty((Ll // 64,), dtype=np.int32)
    _lib().orc_gather_virtual_kv(_p(kp), B, H, S, Lp // S, d, _p(src), nl, _p(cos), _p(sin), rot_offset,
                                 2 * cos.shape[1], rows_per_block, _p(k8), _p(ks), _p(vbs))
    return k8, ks, vbs


def run(wl, sel=None, tau=None):
    """The whole path for one workload: quantize Q (128-row blocks) and K
    (k_scale_rows blocks, or the virtual-KV gather), quantize V when it is an
    INT8 cache, route, then the forward pass over ``sel``."""
    tau = wl.threshold if tau is None else tau
    if wl.qk_float and (wl.virtual or wl.v_int8):
        raise ValueError("the floating QK path takes bf16 Q, K and V")
    q8, qs = quantize(wl.q, wl.lq_valid, 128)
    vbs = None
    if wl.virtual:
        k8, ks, vbs = gather_virtual_kv(wl.k, wl.rows_per_slice, wl.src_map, wl.rope_cos, wl.rope_sin,
                                        wl.rot_offset, wl.k_scale_rows)
    else:
        k8, ks = quantize(wl.k, wl.lkv_valid, wl.k_scale_rows)
    vkw = {}
    if wl.v_int8:
        # a virtual context's V is its physical slices, all valid
        v8, vs = quantize(wl.v, wl.v.shape[2] if wl.virtual else wl.lkv_valid, wl.v_scale_rows)
        vkw = dict(v8=v8, v_scale=vs, v_scale_rows=wl.v_scale_rows)
    else:
        vkw = dict(v_bits=wl.v)
    r = route(q8, k8, ks, wl.k_scale_rows, wl.lq_valid, wl.lkv_valid, v_block_src=vbs, tau=tau,
              G=wl.centroids_per_block, prefix=wl.prefix_tokens, kblock=wl.kblock,
              explicit_map=wl.explicit_map, map_kblock=wl.map_kblock, rule=wl.rule, sparsity=wl.sparsity,
              segments=wl.segments, **vkw)
    out, lse, sel = forward(q8, qs, k8, ks, wl.k_scale_rows, wl.lq_valid, wl.lkv_valid, r["map"],
                            kbar=r["kbar"], vbar=r["vbar"], count=r["count"], v_block_src=vbs,
                            kblock=wl.kblock, G=wl.centroids_per_block, sm_scale=wl.sm_scale, sel=sel,
                            segments=wl.segments, q_bits=wl.q if wl.qk_float else None,
                            k_bits=wl.k if wl.qk_float else None, **vkw)
    return dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, v_block_src=vbs, out=out, lse=lse, sel=sel, **r,
                **{k: v for k, v in vkw.items() if k != "v_bits"})
