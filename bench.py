"""Benchmark of one block-sparse INT8 attention forward on one MI355X.

A step is the whole per-call path on one stream, inputs already resident in HBM:
quantize_qk_int8(Q, 128-row blocks) -> quantize_qk_int8(K, 64-row blocks) ->
sparse_attn_route (Sol 1x64, threshold 1.0; or the fixed-sparsity rule with
--rule topk) -> sparse_attn_fwd.
Workload: B=1, H=40, d=128, L=32768 (21 frames x 30x52 = 32760 valid tokens +
8 padding rows), per-frame low-rank correlated bf16 Q/K/V (synthetic, seeded).

Prints one JSON line.  value = dense-equivalent TOPS = 4*B*H*L*L*d / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attn fwd ms + dense-equiv TOPS, L=32K H=40 d=128, 1x64 thr=1.0"
# MI355X published dense peaks (TFLOP/s or TOP/s) and HBM bandwidth (GB/s)
PEAK_INT8 = 5000.0
PEAK_BF16 = 2500.0
PEAK_HBM = 8000.0
FWD_KERNEL_SOURCES = ["block_sparse_int8_amd/csrc/fwd.hip", "block_sparse_int8_amd/csrc/sa_device.h",
                      "block_sparse_int8_amd/csrc/sa_launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_wan14b_c3_traffic.txt")


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in FWD_KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(expect_hash: str):
    """HBM bytes per fwd launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on another version of the kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_hash") != expect_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fwd_algorithmic_ops(bmap: np.ndarray, count: np.ndarray, d: int) -> tuple:
    """Ops the method itself performs in the forward kernel: per exact
    (128-query x 64-key) tile 2*128*64*d for QK^T and as many for PV; per
    centroid column with a non-zero count 2*128*d + 2*128*d.  Returns
    (ops, exact tiles, centroid columns)."""
    exact_tiles = float((bmap == 1).sum())
    cen = (bmap == 2)
    # columns: per centroid block, the groups with count > 0
    nz = (count > 0).sum(axis=-1)                      # [B,H,nKB]
    cols = float((cen * nz[:, :, None, :]).sum())
    return exact_tiles * 4.0 * 128 * 64 * d + cols * 4.0 * 128 * d, exact_tiles, cols


def cpu_baseline(wl, sample_stride: int):
    """Time the oracle (as it stands) on the host cores: quantize Q and K and
    route in full, the forward pass on every sample_stride-th query block,
    extrapolated to the whole workload."""
    import oracle
    t0 = time.perf_counter()
    q8, qs = oracle.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = oracle.quantize(wl.k, wl.lkv_valid, 64)
    t1 = time.perf_counter()
    r = oracle.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=wl.threshold, G=1, kblock=64,
                     rule=wl.rule, sparsity=wl.sparsity)
    t2 = time.perf_counter()
    nQB = wl.Lq // 128
    total = wl.B * wl.H * nQB
    sel = np.arange(0, total, sample_stride, dtype=np.int64)
    out, lse, _ = oracle.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                                 vbar=r["vbar"], count=r["count"], v_bits=wl.v, kblock=64, G=1,
                                 sm_scale=wl.sm_scale, sel=sel, q_bits=wl.q if wl.qk_float else None,
                                 k_bits=wl.k if wl.qk_float else None)
    t3 = time.perf_counter()
    fwd_full = (t3 - t2) * total / len(sel)
    est = (t1 - t0) + (t2 - t1) + fwd_full
    return dict(est_s=est, quant_s=t1 - t0, route_s=t2 - t1, fwd_sample_s=t3 - t2, nsel=len(sel), total=total,
                threads=oracle.num_threads(), sel=sel, out=out, map=r["map"], tie=r["tie"])


def bench_cache_append(args, sa, W):
    """Streaming INT8 cache: append the newest frame's K and V (12 heads x 2048
    rows x 128) into rings of 64 slabs (four frames), and a whole four-frame
    chunk.  One JSON line; value = HBM bytes the appends must move / time."""
    import torch
    H, d, F, slots = 12, 128, 2048, 64
    rng = np.random.default_rng(2)
    frames = torch.from_numpy(W.bf16_bits(rng.standard_normal((1, H, 4 * F, d), dtype=np.float32)).view(np.int16))
    k = frames.view(torch.bfloat16).cuda()
    v = k.flip(2).contiguous()
    kq = torch.zeros((1, H, slots * 128, d), dtype=torch.int8, device="cuda")
    ks = torch.zeros((1, H, slots), dtype=torch.float32, device="cuda")
    vq, vs = torch.zeros_like(kq), torch.zeros_like(ks)
    stream = torch.cuda.current_stream()

    def run(rows, reps):
        """us per append (one tensor), timed over replays of a captured HIP graph
        of `reps` K and V appends so host launch overhead is not in the time."""
        slot = 0
        for _ in range(args.warmup):
            sa.kv_cache_append_int8(k[:, :, :rows], kq, ks, slot)
            slot = sa.kv_cache_append_int8(v[:, :, :rows], vq, vs, slot)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                s_ = slot
                for _ in range(reps):
                    sa.kv_cache_append_int8(k[:, :, :rows], kq, ks, s_, stream=side)
                    s_ = sa.kv_cache_append_int8(v[:, :, :rows], vq, vs, s_, stream=side)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (2 * reps)

    reps = max(args.steps, 1) * 20
    t1, t4 = run(F, reps), run(4 * F, reps)
    per = lambda rows: H * rows * d * 3 + H * (rows // 128) * 4
    res = {"metric": "streaming INT8 K/V cache append GB/s (FlashVSR-like: H=12, d=128, 2048-row frames)",
           "value": round(per(4 * F) / (t4 * 1e-6) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 in, int8 + fp32 scale out", "data": "synthetic (seeded N(0,1) bf16)",
           "config": {"workload": "kv_cache_append_int8 of K and V into rings of 64 slabs of 128 rows",
                      "H": H, "d": d, "frame_rows": F, "slots": slots},
           "us_per_append": {"one_frame": round(t1, 2), "four_frames": round(t4, 2)},
           "GB/s": {"one_frame": round(per(F) / (t1 * 1e-6) / 1e9, 1),
                    "four_frames": round(per(4 * F) / (t4 * 1e-6) / 1e9, 1)},
           "frac_of_8TB/s": round(per(4 * F) / (t4 * 1e-6) / 1e9 / PEAK_HBM, 4)}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-stride", type=int, default=40)
    ap.add_argument("--heads", type=int, default=40, help="heads (40 for the measured workload)")
    ap.add_argument("--rule", choices=["threshold", "topk"], default="threshold",
                    help="routing rule: Sol threshold 1.0 (the measured workload) or fixed sparsity")
    ap.add_argument("--sparsity", type=float, default=0.75, help="pruned fraction for --rule topk")
    ap.add_argument("--qk-float", action="store_true",
                    help="exact tiles on the floating path (bf16 QK^T) instead of INT8 (same map and centroids)")
    ap.add_argument("--cache-append", action="store_true",
                    help="measure the streaming INT8 K/V cache append instead (FlashVSR-like: H=12, frames of "
                         "2048 rows, a ring of four frames)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (scales HBM counters under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path runs on one MI355X); --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_int8_amd as sa
    import workloads as W

    sa.device_check(0)
    if args.cache_append:
        bench_cache_append(args, sa, W)
        return
    t = time.perf_counter()
    wl = W.wan_like(H=args.heads)
    topk = args.rule == "topk"
    if topk:
        wl.rule, wl.sparsity = 1, args.sparsity
    wl.qk_float = args.qk_float
    log(f"[bench] generated {wl.name}: B={wl.B} H={wl.H} L={wl.Lq} d={wl.d} in {time.perf_counter() - t:.1f}s")
    q, k, v = bf16_dev(wl.q), bf16_dev(wl.k), bf16_dev(wl.v)
    B, H, L, d = q.shape
    nQB, nKB = L // 128, L // 64
    dev = q.device
    stream = torch.cuda.current_stream()
    # outputs and workspace allocated once, outside the timed region
    q8 = torch.empty((B, H, L, d), dtype=torch.int8, device=dev)
    qs = torch.empty((B, H, nQB), dtype=torch.float32, device=dev)
    k8 = torch.empty((B, H, L, d), dtype=torch.int8, device=dev)
    ks = torch.empty((B, H, nKB), dtype=torch.float32, device=dev)
    routed = dict(map=torch.empty((B, H, nQB, nKB), dtype=torch.uint8, device=dev),
                  k_centroid=torch.empty((B, H, nKB, 1, d), dtype=torch.float32, device=dev),
                  v_centroid=torch.empty((B, H, nKB, 1, d), dtype=torch.float32, device=dev),
                  count=torch.empty((B, H, nKB, 1), dtype=torch.float32, device=dev))
    out = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=dev)
    ws = None

    def step(ev=None):
        nonlocal ws
        if ev: ev[0].record(stream)
        sa.quantize_qk_int8(q, wl.lq_valid, 128, out=q8, scale=qs)
        if ev: ev[1].record(stream)
        sa.quantize_qk_int8(k, wl.lkv_valid, 64, out=k8, scale=ks)
        if ev: ev[2].record(stream)
        r = sa.sparse_attn_route(q8, k8, ks, v, lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid,
                                 threshold=wl.threshold, centroids_per_block=1, kblock=64, workspace=ws,
                                 rule=wl.rule, sparsity=wl.sparsity, outputs=routed)
        ws = r["workspace"]
        if ev: ev[3].record(stream)
        if args.qk_float:
            sa.sparse_attn_fwd_float(q, k, v, routed["map"], k_centroid=routed["k_centroid"],
                                     v_centroid=routed["v_centroid"], count=routed["count"], lq_valid=wl.lq_valid,
                                     lkv_valid=wl.lkv_valid, centroids_per_block=1, kblock=64,
                                     sm_scale=wl.sm_scale, out_dtype=torch.bfloat16, out=out)
        else:
            sa.sparse_attn_fwd(q8, qs, k8, ks, v, routed["map"], k_centroid=routed["k_centroid"],
                               v_centroid=routed["v_centroid"], count=routed["count"], lq_valid=wl.lq_valid,
                               lkv_valid=wl.lkv_valid, centroids_per_block=1, kblock=64, sm_scale=wl.sm_scale,
                               out_dtype=torch.bfloat16, out=out)
        if ev: ev[4].record(stream)

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(4)] for s in range(args.steps)])
    ms_step = wall * 1e3 / args.steps
    stage_ms = stage.mean(axis=0)
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step wall; stages (ms) quantQ {stage_ms[0]:.3f} "
        f"quantK {stage_ms[1]:.3f} route {stage_ms[2]:.3f} fwd {stage_ms[3]:.3f}")

    bmap = routed["map"].cpu().numpy()
    cnt = routed["count"].cpu().numpy()
    ops, exact_tiles, cols = fwd_algorithmic_ops(bmap, cnt, d)
    fwd_ms = float(stage_ms[3])
    achieved = ops / (fwd_ms * 1e-3) / 1e12
    # The exact tiles do as many int8 ops (QK^T) as bf16 flops (PV), so the
    # kernel's ceiling is the harmonic combination of the two peaks.
    peak_mixed = 1.0 / (0.5 / PEAK_INT8 + 0.5 / PEAK_BF16)
    if args.qk_float:
        peak_mixed = PEAK_BF16   # both products on bf16 matrix cores
    khash = kernel_hash()
    traffic = None if args.qk_float else read_traffic(khash)   # counters were taken on the INT8 kernel
    elems = B * H * L * d
    quant_bytes = elems * 2 + elems * 1 + B * H * nQB * 4
    dense_ops = 4.0 * B * H * L * L * d
    value = dense_ops / (ms_step * 1e-3) / 1e12
    valid_blocks = -(-wl.lkv_valid // 64)
    kept = float((bmap[..., :valid_blocks] == 1).mean())
    rule_desc = f"top-k sparsity {wl.sparsity:g}" if topk else f"threshold {wl.threshold:g}"
    res = {
        "metric": (METRIC if not topk else METRIC.replace("thr=1.0", f"top-k sparsity={wl.sparsity:g}"))
                  + (", bf16 QK" if args.qk_float else ""),
        "value": round(value, 3),
        "unit": "dense-equiv TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 QK^T + fp32 softmax + bf16 PV" if args.qk_float else "int8 QK^T + fp32 softmax + bf16 PV",
        "data": "synthetic (seeded per-frame low-rank correlated bf16 Q/K/V)",
        "config": {"workload": f"Wan-14B-like Sol 1x64: B=1 H={H} d=128 L=32768 (32760 valid), {rule_desc}",
                   "B": B, "H": H, "L": L, "d": d, "valid": wl.lkv_valid, "kblock": 64, "centroids": "1x64",
                   "rule": args.rule, "threshold": wl.threshold, "sparsity": wl.sparsity if topk else None,
                   "out_dtype": "bf16", "parallelism": "single GPU"},
        "stages_ms": {"quantize_q": round(float(stage_ms[0]), 4), "quantize_k": round(float(stage_ms[1]), 4),
                      "route": round(float(stage_ms[2]), 4), "fwd": round(fwd_ms, 4)},
        "routing": {"kept_fraction": round(kept, 5), "exact_tiles": int(exact_tiles), "centroid_columns": int(cols),
                    "map_entries": int(bmap.size)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak_mixed, 2),
                     "unit": "TFLOP/s", "frac": round(achieved / peak_mixed, 4), "traffic": traffic,
                     "kernel": ("sparse_attn_fwd_float (fwd_kernel<128,true,false,true>)" if args.qk_float
                                else "sparse_attn_fwd (fwd_kernel<128,false,false,true>)"),
                     "frac_of_int8_peak": round(achieved / PEAK_INT8, 4), "kernel_hash": khash},
        "hbm_kernels": {
            "quantize_qk_int8": {"bytes": quant_bytes,
                                 "GB/s": round(quant_bytes / (0.5 * (stage_ms[0] + stage_ms[1]) * 1e-3) / 1e9, 1),
                                 "frac_of_8TB/s": round(quant_bytes / (0.5 * (stage_ms[0] + stage_ms[1]) * 1e-3)
                                                        / 1e9 / PEAK_HBM, 4)},
        },
    }
    route_bytes = elems * 1 * 2 + elems * 2 + B * H * nKB * d * 4 * 2 + bmap.size
    res["hbm_kernels"]["sparse_attn_route"] = {
        "bytes": route_bytes, "GB/s": round(route_bytes / (stage_ms[2] * 1e-3) / 1e9, 1),
        "frac_of_8TB/s": round(route_bytes / (stage_ms[2] * 1e-3) / 1e9 / PEAK_HBM, 4)}

    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on a sample (every {args.cpu_sample_stride}th query block) ...")
        cb = cpu_baseline(wl, args.cpu_sample_stride)
        cpu_tops = dense_ops / cb["est_s"] / 1e12
        res["cpu_baseline"] = {
            "value": round(cpu_tops, 6), "unit": "dense-equiv TOPS", "cores": cb["threads"], "kind": "oracle",
            "sample": (f"quantize Q/K and route over the whole workload ({cb['quant_s'] + cb['route_s']:.1f}s), "
                       f"forward on {cb['nsel']} of {cb['total']} query blocks (every "
                       f"{args.cpu_sample_stride}th, {cb['fwd_sample_s']:.1f}s) scaled by {cb['total'] / cb['nsel']:.0f}x; "
                       f"estimated {cb['est_s']:.1f}s per forward"),
            "ms_per_step_est": round(cb["est_s"] * 1e3, 1)}
        # spot parity on the sampled blocks (same inputs, maps compared first)
        gout = out.float().cpu().numpy().reshape(B * H, L, d)
        mism = int(((bmap != cb["map"]) & (cb["tie"] == 0)).sum())
        errs = []
        for e, sid in enumerate(cb["sel"]):
            bh, i = divmod(int(sid), nQB)
            if (bmap.reshape(B * H, nQB, nKB)[bh, i] != cb["map"].reshape(B * H, nQB, nKB)[bh, i]).any():
                continue
            r1 = min(128, max(0, wl.lq_valid - i * 128))
            errs.append(np.abs(gout[bh, i * 128:i * 128 + r1] - cb["out"][e, :r1]).reshape(-1))
        e = np.concatenate(errs) if errs else np.zeros(1)
        res["parity_sample"] = {"map_mismatches_outside_ties": mism, "ties": int(cb["tie"].sum()),
                                "max_abs": float(e.max()), "mean_abs": float(e.mean()), "out_dtype": "bf16"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
