"""Shared helpers for the GPU parity tests: run a workload through the HIP path
(via the C ABI binding) and through the oracle on the same seeded inputs, and
compare them at the bars the method fixes:

  * INT8 codes, scales, virtual-KV tables: bit-exact
  * block maps: bit-exact except entries the oracle flags as ties
    (|s - threshold| <= 1e-6 sigma), which are counted
  * outputs: max-abs <= 1e-2 and mean-abs <= 1e-3 over valid rows
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def gpu_pipeline(wl, tau=None, out_dtype=torch.float32, kblock=None, map_kblock=None, G=None, sums=True):
    """The whole HIP path for one workload.  Returns host numpy arrays.
    ``sums``: the quantizer also writes the codes' column sums and the route
    takes them (as bench.py and sparse_attention run it); False: the route
    sums the codes itself."""
    import block_sparse_int8_amd as sa
    tau = wl.threshold if tau is None else tau
    kblock = wl.kblock if kblock is None else kblock
    G = wl.centroids_per_block if G is None else G
    q = bf16_dev(wl.q)
    k = bf16_dev(wl.k)
    v = bf16_dev(wl.v)
    qsum = ksum = None
    if sums:
        q8, qs, qsum = sa.quantize_qk_int8(q, wl.lq_valid, 128, col_sums=True, sum_rows=128)
    else:
        q8, qs = sa.quantize_qk_int8(q, wl.lq_valid, 128)
    vbs = None
    if wl.virtual:
        cos = torch.from_numpy(wl.rope_cos).cuda()
        sin = torch.from_numpy(wl.rope_sin).cuda()
        k8, ks, vbs = sa.gather_virtual_kv(k, wl.rows_per_slice, wl.src_map.tolist(), cos, sin, wl.rot_offset,
                                           wl.k_scale_rows)
    elif sums:
        k8, ks, ksum = sa.quantize_qk_int8(k, wl.lkv_valid, wl.k_scale_rows, col_sums=True, sum_rows=32)
    else:
        k8, ks = sa.quantize_qk_int8(k, wl.lkv_valid, wl.k_scale_rows)
    v_in, vsc = v, None
    if wl.v_int8:
        # a virtual context's V is its physical slices, all valid
        v_in, vsc = sa.quantize_qk_int8(v, wl.v.shape[2] if wl.virtual else wl.lkv_valid, wl.v_scale_rows)
    em = None
    if wl.explicit_map is not None:
        em = torch.from_numpy(np.ascontiguousarray(wl.explicit_map)).cuda()
    r = sa.sparse_attn_route(q8, k8, ks, v_in, lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid, v_scale=vsc,
                             v_block_src=vbs, threshold=tau, centroids_per_block=G,
                             prefix_tokens=wl.prefix_tokens, kblock=kblock, k_scale_rows=wl.k_scale_rows,
                             v_scale_rows=wl.v_scale_rows, explicit_map=em,
                             map_kblock=map_kblock or wl.map_kblock, rule=wl.rule, sparsity=wl.sparsity,
                             segments=wl.segments, row_stats=True, q_sums=qsum, k_sums=ksum)
    if wl.qk_float:
        out, lse = sa.sparse_attn_fwd_float(q, k, v, r["map"], k_centroid=r["k_centroid"],
                                            v_centroid=r["v_centroid"], count=r["count"], lq_valid=wl.lq_valid,
                                            lkv_valid=wl.lkv_valid, centroids_per_block=G, kblock=kblock,
                                            sm_scale=wl.sm_scale, out_dtype=out_dtype, return_lse=True,
                                            segments=wl.segments)
    else:
        out, lse = sa.sparse_attn_fwd(q8, qs, k8, ks, v_in, r["map"], k_centroid=r["k_centroid"],
                                      v_centroid=r["v_centroid"], count=r["count"], lq_valid=wl.lq_valid,
                                      lkv_valid=wl.lkv_valid, v_scale=vsc, v_block_src=vbs, centroids_per_block=G,
                                      kblock=kblock, k_scale_rows=wl.k_scale_rows, v_scale_rows=wl.v_scale_rows,
                                      sm_scale=wl.sm_scale, out_dtype=out_dtype, return_lse=True,
                                      segments=wl.segments)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy()
    res = dict(q8=host(q8), q_scale=host(qs), k8=host(k8), k_scale=host(ks), map=host(r["map"]),
               kbar=host(r["k_centroid"]), vbar=host(r["v_centroid"]), count=host(r["count"]),
               stats=host(r["row_stats"]), out=out.float().cpu().numpy(), lse=host(lse),
               v_block_src=host(vbs))
    if wl.v_int8:
        res["v8"], res["v_scale"] = host(v_in), host(vsc)
    res["q_sums"], res["k_sums"] = host(qsum), host(ksum)
    return res


def compare_maps(g_map, o_map, o_tie):
    """Returns (mismatches outside ties, tie count, tie mismatches)."""
    diff = g_map != o_map
    tie = o_tie.astype(bool)
    return int((diff & ~tie).sum()), int(tie.sum()), int((diff & tie).sum())


def compare_outputs(g_out, o_out, sel, nQB, Lq, lq_valid, skip_blocks=()):
    """g_out [B,H,Lq,d]; o_out [nsel,128,d] for selected blocks.  Returns
    (max_abs, mean_abs, rows compared)."""
    B_H = g_out.shape[0] * g_out.shape[1]
    g = g_out.reshape(B_H, Lq, -1)
    errs = []
    rows = 0
    for e, sid in enumerate(np.asarray(sel)):
        if int(sid) in skip_blocks:
            continue
        bh, i = divmod(int(sid), nQB)
        r1 = min(128, max(0, lq_valid - i * 128))
        if r1 == 0:
            continue
        d = np.abs(g[bh, i * 128:i * 128 + r1] - o_out[e, :r1])
        errs.append(d)
        rows += r1
        # padded rows must be exactly zero
        assert not g[bh, i * 128 + r1:(i + 1) * 128].any()
    if not errs:
        return 0.0, 0.0, 0
    allerr = np.concatenate([x.reshape(-1) for x in errs])
    return float(allerr.max()), float(allerr.mean()), rows


def tie_blocks(g_map, o_map, nQB):
    """Query blocks (flat ids) whose map rows differ (only at ties)."""
    B, H = g_map.shape[:2]
    bad = (g_map != o_map).any(axis=-1).reshape(-1)
    return set(np.nonzero(bad)[0].tolist())


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        say(f"  [{self.what}: {time.time() - self.t:.1f}s]")
