"""The allocation-free routing entry point (sparse_attn_route_noalloc).

For callers that cannot allocate device memory (HIP graph capture, tight
serving loops): the same routing pass as sparse_attn_route, with the block sums
in the library's own per-device array instead of a caller workspace.  Checked
through the C ABI against sparse_attn_route on two calls in a row, the second
with a smaller input (the array keeps the first call's contents), under both
routing rules; and, on the host, that shapes needing more than the array are
refused before anything is queued.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_int8_amd as sa
import workloads as W
from tests.helpers import bf16_dev, say


def _route_inputs(wl):
    q, k, v = bf16_dev(wl.q), bf16_dev(wl.k), bf16_dev(wl.v)
    q8, _ = sa.quantize_qk_int8(q, wl.lq_valid, 128)
    k8, ks = sa.quantize_qk_int8(k, wl.lkv_valid, wl.kblock)
    return q8, k8, ks, v


def _outputs(wl):
    B, H, Lq, d = wl.q.shape
    nQB, nKB, G = Lq // 128, wl.Lkv // wl.kblock, wl.centroids_per_block
    dev = "cuda"
    return dict(map=torch.empty((B, H, nQB, nKB), dtype=torch.uint8, device=dev),
                k_centroid=torch.empty((B, H, nKB, G, d), dtype=torch.float32, device=dev),
                v_centroid=torch.empty((B, H, nKB, G, d), dtype=torch.float32, device=dev),
                count=torch.empty((B, H, nKB, G), dtype=torch.float32, device=dev),
                row_stats=torch.empty((B, H, nQB, 2), dtype=torch.float64, device=dev))


@pytest.mark.gpu
def test_noalloc_route_matches_route_on_two_calls():
    assert torch.cuda.is_available()
    sa.device_check(torch.cuda.current_device())
    big = W.config(3, small=True)                      # 2 heads, 3968 rows, threshold rule
    small = W.tiny_sol(seed=44, H=2, L=640, d=128, valid=600, centroids_per_block=2)
    small.rule, small.sparsity = 1, 0.6                 # second call: smaller, fixed sparsity
    for n, wl in enumerate((big, small)):
        say(f"case noalloc call {n + 1}: {wl.name} H={wl.H} L={wl.Lq} d={wl.d} rule={wl.rule}")
        q8, k8, ks, v = _route_inputs(wl)
        kw = dict(lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid, threshold=wl.threshold,
                  centroids_per_block=wl.centroids_per_block, kblock=wl.kblock, rule=wl.rule,
                  sparsity=wl.sparsity, row_stats=True)
        ref = sa.sparse_attn_route(q8, k8, ks, v, **kw)
        got = sa.sparse_attn_route_noalloc(q8, k8, ks, v, outputs=_outputs(wl), **kw)
        torch.cuda.synchronize()
        assert got["workspace"] is None
        for key in ("map", "k_centroid", "v_centroid", "count", "row_stats"):
            a, b = got[key].cpu().numpy(), ref[key].cpu().numpy()
            assert np.array_equal(a, b, equal_nan=True), key
        say(f"  map {int((got['map'] == 1).sum().item())} exact / {int((got['map'] == 2).sum().item())} centroid")


def test_noalloc_refuses_shapes_beyond_the_array():
    """Host only: a call whose workspace would exceed SA_ROUTE_SCRATCH_BYTES
    (16 MiB) fails with SA_E_WORKSPACE and a message naming the limit, before
    any device work (no pointer is touched)."""
    lib = sa.load()
    # 128 heads at L = 32768, d = 128: 24 MiB of block sums
    dims = sa.sa_dims(1, 128, 32768, 32768, 128, 32768, 32768, 32768)
    prm = sa._params(1.0, 1, 0, 64, 64, 128, 64)
    assert lib.sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 0) > 16 << 20
    fake = ctypes.c_void_p(1 << 20)         # never dereferenced: validation fails first
    rc = lib.sparse_attn_route_noalloc(fake, fake, fake, fake, sa.SA_BF16, None, None, None, None,
                                       ctypes.byref(dims), ctypes.byref(prm), None, fake, fake, fake, fake, None, None)
    assert rc == sa.SA_E_WORKSPACE
    msg = lib.sa_last_error().decode()
    assert "sparse_attn_route_noalloc" in msg and str(16 << 20) in msg
