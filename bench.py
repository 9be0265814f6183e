"""Benchmark of one block-sparse INT8 attention forward on one MI355X.

A step is the whole per-call path on one stream, inputs already resident in HBM:
quantize_qk_int8(Q, 128-row blocks) -> the K side (quantize_qk_int8(K), the
INT8 K/V cache append, or the virtual-KV gather) -> sparse_attn_route ->
sparse_attn_fwd.  The default workload is the measured one:
B=1, H=40, d=128, L=32768 (21 frames x 30x52 = 32760 valid tokens + 8 padding
rows), per-frame low-rank correlated bf16 Q/K/V (synthetic, seeded), Sol 1x64
threshold 1.0.  --config 1..5 picks the other workloads (--config all: one line
each).

Timing: W warm-up steps, then exactly K back-to-back steps between two device
synchronizations (ms_per_step, value); HIP events on the same stream bracket
every stage (their means give the roofline figures).  Then K more steps, each
after an untimed 1 GiB write that evicts the 256 MB last-level cache, timed by
events alone: medians with p10 and p90 per stage ("stages_cold_ms").

After the timed steps a probe kernel measures this GPU's sustained
matrix-core rate for the forward's op mix on random operands; the roofline
object gives the forward's fraction of it beside the datasheet fractions.

Prints one JSON line per workload.  value = dense-equivalent TOPS =
4*B*H*Lq*Lkv*d / step time.  --peaks prints the measured matrix-core and HBM
ceilings instead.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
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
FLUSH_BYTES = 1 << 30


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


def fwd_algorithmic_ops(bmap: np.ndarray, count: np.ndarray, d: int, kblock: int = 64) -> tuple:
    """Ops the method itself performs in the forward kernel: per exact
    (128-query x 64-key) tile 2*128*64*d for QK^T and as many for PV (a key
    block of kblock rows is kblock/64 tiles); per centroid column with a
    non-zero count 2*128*d + 2*128*d.  Returns (ops, exact tiles, centroid
    columns)."""
    exact_tiles = float((bmap == 1).sum()) * (kblock // 64)
    cols = 0.0
    if count is not None:
        cen = (bmap == 2)
        nz = (count > 0).sum(axis=-1)                      # [B,H,nKB]
        cols = float((cen * nz[:, :, None, :]).sum())
    return exact_tiles * 4.0 * 128 * 64 * d + cols * 4.0 * 128 * d, exact_tiles, cols


def host_info():
    """CPU model and logical CPU count of this host."""
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def stats(x):
    x = np.asarray(x, dtype=np.float64)
    return {"median": round(float(np.median(x)), 4), "p10": round(float(np.percentile(x, 10)), 4),
            "p90": round(float(np.percentile(x, 90)), 4)}


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

class Case:
    """One workload on the device: inputs, preallocated outputs, its stages
    (name -> callable) in order, the algorithmic bytes of each HBM-bound stage
    and everything the report needs."""

    def __init__(self, n, args, sa, W, torch):
        self.n, self.sa, self.torch = n, sa, torch
        t = time.perf_counter()
        if n == 3:
            wl = W.wan_like(H=args.heads)
        elif n == SEG:
            wl = W.ref2va_segments()
        else:
            wl = W.config(n)
        if args.rule == "topk" and wl.explicit_map is None:
            wl.rule, wl.sparsity = 1, args.sparsity
        wl.qk_float = bool(args.qk_float)
        if wl.qk_float and wl.v_int8:
            raise SystemExit("--qk-float needs bf16 V (not the INT8 cache workload)")
        self.wl = wl
        log(f"[bench] generated {wl.name}: B={wl.B} H={wl.H} Lq={wl.Lq} Lkv={wl.Lkv} d={wl.d} "
            f"in {time.perf_counter() - t:.1f}s")
        dev = torch.device("cuda")
        bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        self.q, self.k, self.v = bf(wl.q), bf(wl.k), bf(wl.v)
        B, H, Lq, d = self.q.shape
        Lkv, kb, G = wl.Lkv, wl.kblock, wl.centroids_per_block
        nQB, nKB = Lq // 128, Lkv // kb
        self.B, self.H, self.Lq, self.Lkv, self.d, self.kb, self.G = B, H, Lq, Lkv, d, kb, G
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.q8, self.qs = e((B, H, Lq, d), torch.int8), e((B, H, nQB), torch.float32)
        self.k8, self.ks = e((B, H, Lkv, d), torch.int8), e((B, H, Lkv // wl.k_scale_rows), torch.float32)
        self.vbs = None
        self.v_in, self.vsc = self.v, None
        if wl.v_int8:
            self.v8, self.vsc = e((B, H, Lkv, d), torch.int8), e((B, H, Lkv // wl.v_scale_rows), torch.float32)
            self.v_in = self.v8
        if wl.virtual:
            self.cos = torch.from_numpy(wl.rope_cos).to(dev)
            self.sin = torch.from_numpy(wl.rope_sin).to(dev)
        Gs = max(G, 1)
        self.routed = dict(map=e((B, H, nQB, nKB), torch.uint8), k_centroid=e((B, H, nKB, Gs, d), torch.float32),
                           v_centroid=e((B, H, nKB, Gs, d), torch.float32), count=e((B, H, nKB, Gs), torch.float32))
        if G == 0:
            self.routed = dict(map=self.routed["map"])
        self.em = None if wl.explicit_map is None else torch.from_numpy(np.ascontiguousarray(wl.explicit_map)).to(dev)
        self.out = e((B, H, Lq, d), torch.bfloat16)
        self.ws = None
        self.stage_names = ["quantize_q", "k_side", "route", "fwd"]
        # the quantizer writes the codes' column sums and the route reads them
        # instead of the codes (routing rules and centroids need the sums)
        self.use_sums = wl.explicit_map is None or G > 0
        self.qsum = e((B, H, Lq // 128, d), torch.int16) if wl.explicit_map is None else None
        self.ksum = (e((B, H, Lkv // 32, d), torch.int16) if self.use_sums and not wl.virtual and not wl.v_int8
                     else None)

    # -- stages ---------------------------------------------------------------
    def quantize_q(self):
        self.sa.quantize_qk_int8(self.q, self.wl.lq_valid, 128, out=self.q8, scale=self.qs,
                                 col_sums=self.qsum if self.qsum is not None else False, sum_rows=128)

    def k_side(self):
        wl, sa = self.wl, self.sa
        if wl.virtual:
            kq, ks, vbs = sa.gather_virtual_kv(self.k, wl.rows_per_slice, wl.src_map.tolist(), self.cos, self.sin,
                                               wl.rot_offset, wl.k_scale_rows)
            self.k8, self.ks, self.vbs = kq, ks, vbs
            return
        if wl.v_int8:
            # FlashVSR: K and V kept as an INT8 cache of 128-row slabs; the whole
            # cache is (re)written here, as the streaming append would over time
            sa.kv_cache_append_int8(self.k, self.k8, self.ks, 0, wl.lkv_valid, wl.k_scale_rows)
            sa.kv_cache_append_int8(self.v, self.v8, self.vsc, 0, wl.lkv_valid, wl.v_scale_rows)
            return
        sa.quantize_qk_int8(self.k, wl.lkv_valid, wl.k_scale_rows, out=self.k8, scale=self.ks,
                            col_sums=self.ksum if self.ksum is not None else False, sum_rows=32)

    def route(self):
        wl = self.wl
        r = self.sa.sparse_attn_route(self.q8, self.k8, self.ks, self.v_in, lq_valid=wl.lq_valid,
                                      lkv_valid=wl.lkv_valid, v_scale=self.vsc, v_block_src=self.vbs,
                                      threshold=wl.threshold, centroids_per_block=self.G,
                                      prefix_tokens=wl.prefix_tokens, kblock=self.kb, k_scale_rows=wl.k_scale_rows,
                                      v_scale_rows=wl.v_scale_rows, explicit_map=self.em, map_kblock=wl.map_kblock,
                                      rule=wl.rule, sparsity=wl.sparsity, workspace=self.ws, outputs=self.routed,
                                      q_sums=self.qsum if wl.explicit_map is None else None, k_sums=self.ksum,
                                      segments=wl.segments)
        self.ws = r["workspace"]

    def fwd(self, out_dtype=None, out=None):
        wl, r = self.wl, self.routed
        kw = dict(k_centroid=r.get("k_centroid"), v_centroid=r.get("v_centroid"), count=r.get("count"),
                  lq_valid=wl.lq_valid, lkv_valid=wl.lkv_valid, centroids_per_block=self.G, kblock=self.kb,
                  sm_scale=wl.sm_scale, out_dtype=out_dtype or self.torch.bfloat16,
                  out=self.out if out is None else out, segments=wl.segments)
        if wl.qk_float:
            self.sa.sparse_attn_fwd_float(self.q, self.k, self.v, r["map"], v_block_src=self.vbs, **kw)
        else:
            self.sa.sparse_attn_fwd(self.q8, self.qs, self.k8, self.ks, self.v_in, r["map"], v_scale=self.vsc,
                                    v_block_src=self.vbs, k_scale_rows=wl.k_scale_rows,
                                    v_scale_rows=wl.v_scale_rows, **kw)

    def stages(self):
        return [self.quantize_q, self.k_side, self.route, self.fwd]

    # -- bytes of the HBM-bound stages ---------------------------------------
    def hbm_bytes(self):
        """Bytes each HBM-bound stage must move in this design: reads of its
        inputs and writes of its outputs, each once.  The quantizer's column
        sums (int16 per 32 rows, 1/16 of a code tensor) are written by the
        quantizer and read by the route instead of the codes."""
        wl, B, H, d = self.wl, self.B, self.H, self.d
        nQB, nKB = self.Lq // 128, self.Lkv // self.kb
        qe, ke = B * H * self.Lq * d, B * H * self.Lkv * d
        qsum_b = qe // 64 if self.qsum is not None else 0
        ksum_b = ke // 16 if self.ksum is not None else 0
        out = {"quantize_q": qe * 3 + B * H * nQB * 4 + qsum_b}
        if wl.virtual:
            out["k_side"] = B * H * wl.n_phys * wl.rows_per_slice * d * 2 + ke + B * H * (self.Lkv // 64) * 4
        elif wl.v_int8:
            out["k_side"] = 2 * (ke * 3 + B * H * (self.Lkv // 128) * 4)
        else:
            out["k_side"] = ke * 3 + B * H * (self.Lkv // wl.k_scale_rows) * 4 + ksum_b
        map_bytes = B * H * nQB * nKB
        cen = B * H * nKB * self.G * (2 * d + 1) * 4
        v_bytes = B * H * wl.v.shape[2] * d * (1 if wl.v_int8 else 2)
        if wl.explicit_map is None:
            out["route"] = (qsum_b or qe) + (ksum_b or ke) + v_bytes + cen + map_bytes
        elif self.G > 0:
            out["route"] = (ksum_b or ke) + v_bytes + cen + 2 * map_bytes
        else:
            out["route"] = 2 * map_bytes
        return out

    def plain_route_bytes(self):
        """The route's bytes when it reads the int8 codes themselves: int8 Q,
        int8 K and V read, centroids, counts and the map written (the count the
        measurement plan of this path fixes for the route)."""
        wl, B, H, d = self.wl, self.B, self.H, self.d
        nQB, nKB = self.Lq // 128, self.Lkv // self.kb
        qe, ke = B * H * self.Lq * d, B * H * self.Lkv * d
        return qe + ke + B * H * wl.v.shape[2] * d * 2 + B * H * nKB * self.G * (2 * d + 1) * 4 + B * H * nQB * nKB

    def plain_bytes(self):
        """The bytes the measurement plan of this path assigns to quantizing Q
        and K and to the route (int8 Q, int8 K and V read by the route, outputs
        written), for the routed workloads: their sum over the three stages'
        time is the like-for-like HBM figure whichever stage reads what."""
        wl, B, H, d = self.wl, self.B, self.H, self.d
        nQB, nKB = self.Lq // 128, self.Lkv // self.kb
        qe, ke = B * H * self.Lq * d, B * H * self.Lkv * d
        quant = qe * 3 + B * H * nQB * 4 + ke * 3 + B * H * (self.Lkv // wl.k_scale_rows) * 4
        return quant + self.plain_route_bytes()

    def workload_desc(self):
        wl = self.wl
        rule = (f"top-k sparsity {wl.sparsity:g}" if wl.rule == 1 else
                "explicit map" if wl.explicit_map is not None else f"threshold {wl.threshold:g}")
        names = {1: f"tiny Sol 1x64: B=1 H={self.H} d={self.d} L={self.Lq}, {rule}",
                 2: f"FlashVSR LCSA over an INT8 K/V cache: B=1 H={self.H} d={self.d} L={self.Lq}, 128x128 blocks, "
                    f"{rule}",
                 3: f"Wan-14B-like Sol 1x64: B=1 H={self.H} d=128 L=32768 (32760 valid), {rule}",
                 4: f"Sol 2x32 with 1024-token dense prefix: B=1 H={self.H} d=128 L={self.Lq}, {rule}",
                 5: f"virtual KV residual: B=1 H={self.H} d=128 Lq={self.Lq} Lkv={self.Lkv} logical, {rule}",
                 SEG: f"segmented Ref2VA-like layout: B=1 H={self.H} d=128 L={self.Lq} (text, reference image and "
                      f"audio dense; reference video and 8 generated frames routed), {rule}"}
        return names[self.n]


def cpu_baseline(case, stride: int):
    """Time the oracle (as it stands) on the host cores: quantization, the
    K side and the route over the whole workload, the forward pass on every
    stride-th query block, extrapolated to the whole workload."""
    import oracle
    wl = case.wl
    t0 = time.perf_counter()
    q8, qs = oracle.quantize(wl.q, wl.lq_valid, 128)
    vbs = None
    if wl.virtual:
        k8, ks, vbs = oracle.gather_virtual_kv(wl.k, wl.rows_per_slice, wl.src_map, wl.rope_cos, wl.rope_sin,
                                               wl.rot_offset, wl.k_scale_rows)
    else:
        k8, ks = oracle.quantize(wl.k, wl.lkv_valid, wl.k_scale_rows)
    vkw = dict(v_bits=wl.v)
    if wl.v_int8:
        v8, vs = oracle.quantize(wl.v, wl.lkv_valid, wl.v_scale_rows)
        vkw = dict(v8=v8, v_scale=vs, v_scale_rows=wl.v_scale_rows)
    t1 = time.perf_counter()
    r = oracle.route(q8, k8, ks, wl.k_scale_rows, wl.lq_valid, wl.lkv_valid, v_block_src=vbs, tau=wl.threshold,
                     G=wl.centroids_per_block, prefix=wl.prefix_tokens, kblock=wl.kblock,
                     explicit_map=wl.explicit_map, map_kblock=wl.map_kblock, rule=wl.rule, sparsity=wl.sparsity,
                     segments=wl.segments, **vkw)
    t2 = time.perf_counter()
    nQB = wl.Lq // 128
    total = wl.B * wl.H * nQB
    sel = np.arange(0, total, stride, dtype=np.int64)
    out, _, _ = oracle.forward(q8, qs, k8, ks, wl.k_scale_rows, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                               vbar=r["vbar"], count=r["count"], v_block_src=vbs, kblock=wl.kblock,
                               G=wl.centroids_per_block, sm_scale=wl.sm_scale, sel=sel, segments=wl.segments,
                               q_bits=wl.q if wl.qk_float else None, k_bits=wl.k if wl.qk_float else None, **vkw)
    t3 = time.perf_counter()
    fwd_full = (t3 - t2) * total / len(sel)
    est = (t1 - t0) + (t2 - t1) + fwd_full
    return dict(est_s=est, quant_s=t1 - t0, route_s=t2 - t1, fwd_sample_s=t3 - t2, nsel=len(sel), total=total,
                threads=oracle.num_threads(), sel=sel, out=out, map=r["map"], tie=r["tie"])


# workload id of the segmented key layout (--config seg)
SEG = 6
CPU_STRIDE = {1: 1, 2: 1, 3: 40, 4: 24, 5: 1, SEG: 12}


def run_case(n, args, sa, W, torch):
    case = Case(n, args, sa, W, torch)
    stream = torch.cuda.current_stream()
    stages = case.stages()
    ns = len(stages)

    def step(ev=None):
        for i, f in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            f()
        if ev is not None:
            ev[ns].record(stream)

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # phase A: K back-to-back steps between two synchronizations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm = np.array([[evs[s][i].elapsed_time(evs[s][i + 1]) for i in range(ns)] for s in range(args.steps)])
    ms_step = wall * 1e3 / args.steps
    stage_mean = warm.mean(axis=0)
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step wall; stages (ms) " +
        " ".join(f"{nm} {m:.4f}" for nm, m in zip(case.stage_names, stage_mean)))
    # phase B: K steps, each after an untimed write of FLUSH_BYTES
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    for s in range(args.steps):
        flush.fill_(s & 0xFF)
        step(evc[s])
    torch.cuda.synchronize()
    del flush
    cold = np.array([[evc[s][i].elapsed_time(evc[s][i + 1]) for i in range(ns)] for s in range(args.steps)])
    cold_total = cold.sum(axis=1)

    wl = case.wl
    bmap = case.routed["map"].cpu().numpy()
    cnt = case.routed["count"].cpu().numpy() if "count" in case.routed else None
    ops, exact_tiles, cols = fwd_algorithmic_ops(bmap, cnt, case.d, case.kb)
    fwd_ms = float(stage_mean[3])
    achieved = ops / (fwd_ms * 1e-3) / 1e12
    # The exact tiles do as many int8 ops (QK^T) as bf16 flops (PV), so the
    # kernel's ceiling is the harmonic combination of the two peaks.
    peak_mixed = 1.0 / (0.5 / PEAK_INT8 + 0.5 / PEAK_BF16)
    if wl.qk_float:
        peak_mixed = PEAK_BF16   # both products on bf16 matrix cores
    # the same GPU's sustained matrix-core rate for this op mix, measured now
    mode = 1 if wl.qk_float else 2
    measured_peak, _ = probe_mfma(torch, _probe_lib(), mode)
    log(f"[bench] measured ceiling ({MFMA_PROBE_NAMES[mode]}): {measured_peak:.1f}")
    khash = kernel_hash()
    headline = n == 3 and not wl.qk_float and wl.rule == 0 and case.H == 40
    traffic = read_traffic(khash) if headline else None   # counters were taken on the headline workload
    dense_ops = 4.0 * case.B * case.H * case.Lq * case.Lkv * case.d
    value = dense_ops / (ms_step * 1e-3) / 1e12
    nvalid_blocks = -(-wl.lkv_valid // case.kb)
    kept = float((bmap[..., :nvalid_blocks] == 1).mean())
    if n == 3:
        metric = METRIC if wl.rule == 0 else METRIC.replace("thr=1.0", f"top-k sparsity={wl.sparsity:g}")
        if wl.qk_float:
            metric += ", bf16 QK"
    elif n == SEG:
        metric = "sparse attn fwd ms + dense-equiv TOPS, segmented key layout (Ref2VA-like, H=24, d=128)"
    else:
        metric = f"sparse attn fwd ms + dense-equiv TOPS, workload {n} ({W.CONFIG_NAMES[n]})"
    res = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "dense-equiv TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 QK^T + fp32 softmax + bf16 PV" if wl.qk_float else "int8 QK^T + fp32 softmax + bf16 PV",
        "data": "synthetic (seeded bf16 Q/K/V; " + ("per-frame low-rank correlated)" if n in (3, 4) else
                                                    "N(0,1) conditioning segments, per-frame low-rank correlated video)"
                                                    if n == SEG else "N(0,1))"),
        "config": {"workload": case.workload_desc(), "B": case.B, "H": case.H, "Lq": case.Lq, "Lkv": case.Lkv,
                   "d": case.d, "lq_valid": wl.lq_valid, "lkv_valid": wl.lkv_valid, "kblock": case.kb,
                   "centroids": {0: "none", 1: "1x64", 2: "2x32"}[case.G],
                   "rule": "explicit" if wl.explicit_map is not None else ("topk" if wl.rule == 1 else "threshold"),
                   "threshold": wl.threshold if wl.explicit_map is None and wl.rule == 0 else None,
                   "sparsity": wl.sparsity if wl.rule == 1 else None, "out_dtype": "bf16",
                   "parallelism": "single GPU"},
        "stages_ms": {nm: round(float(m), 4) for nm, m in zip(case.stage_names, stage_mean)},
        "stages_cold_ms": {**{nm: stats(cold[:, i]) for i, nm in enumerate(case.stage_names)},
                           "step": stats(cold_total)},
        "routing": {"kept_fraction": round(kept, 5), "exact_tiles": int(exact_tiles), "centroid_columns": int(cols),
                    "map_entries": int(bmap.size)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak_mixed, 2),
                     "unit": "TFLOP/s", "frac": round(achieved / peak_mixed, 4), "traffic": traffic,
                     "kernel": ("sparse_attn_fwd_float (fwd_kernel<%d,true,false,true>)" % case.d if wl.qk_float
                                else "sparse_attn_fwd (fwd_kernel<%d,false,%s,true>)" % (
                                    case.d, "true" if wl.v_int8 else "false")),
                     "ops_per_launch": ops, "fwd_ms_mean": round(fwd_ms, 4),
                     "frac_of_int8_peak": round(achieved / PEAK_INT8, 4),
                     "measured_peak": round(measured_peak, 1),
                     "frac_of_measured_peak": round(achieved / measured_peak, 4),
                     "measured_peak_probe": ("bf16" if wl.qk_float else "50/50 int8/bf16") +
                                            " MFMA loop on random operands, this GPU, after the timed steps",
                     "kernel_hash": khash},
        "hbm_kernels": {},
    }
    for nm, nbytes in case.hbm_bytes().items():
        i = case.stage_names.index(nm)
        gbs = nbytes / (stage_mean[i] * 1e-3) / 1e9
        res["hbm_kernels"][nm] = {"bytes": int(nbytes), "GB/s": round(gbs, 1),
                                  "frac_of_8TB/s": round(gbs / PEAK_HBM, 4)}
    if wl.explicit_map is None and not wl.virtual:
        # the route by the byte count of a route that reads the codes (this one
        # reads the quantizer's column sums instead, so it moves fewer bytes)
        rb = case.plain_route_bytes()
        i = case.stage_names.index("route")
        gbs = rb / (stage_mean[i] * 1e-3) / 1e9
        res["hbm_kernels"]["route"].update({"bytes_if_reading_codes": int(rb), "GB/s_if_reading_codes": round(gbs, 1),
                                            "frac_of_8TB/s_if_reading_codes": round(gbs / PEAK_HBM, 4)})
        nbytes = case.plain_bytes()
        ms3 = float(stage_mean[0] + stage_mean[1] + stage_mean[2])
        gbs = nbytes / (ms3 * 1e-3) / 1e9
        res["hbm_kernels"]["quantize_q+k_side+route"] = {"bytes": int(nbytes), "ms": round(ms3, 4),
                                                         "GB/s": round(gbs, 1), "frac_of_8TB/s": round(gbs / PEAK_HBM, 4)}

    if not args.no_cpu_baseline:
        stride = args.cpu_sample_stride or CPU_STRIDE[n]
        log(f"[bench] timing the CPU oracle on a sample (every {stride}th query block) ...")
        cb = cpu_baseline(case, stride)
        model, ncpu = host_info()
        res["cpu_baseline"] = {
            "value": round(dense_ops / cb["est_s"] / 1e12, 6), "unit": "dense-equiv TOPS", "cores": cb["threads"],
            "kind": "oracle", "cpu_model": model, "nproc": ncpu,
            "sample": (f"quantize, K side and route over the whole workload ({cb['quant_s'] + cb['route_s']:.1f}s), "
                       f"forward on {cb['nsel']} of {cb['total']} query blocks (every {stride}th, "
                       f"{cb['fwd_sample_s']:.1f}s) scaled by {cb['total'] / cb['nsel']:.0f}x; "
                       f"estimated {cb['est_s']:.1f}s per forward"),
            "ms_per_step_est": round(cb["est_s"] * 1e3, 1)}
        # spot parity on the sampled blocks (same inputs, maps compared first)
        B, H, Lq, d = case.B, case.H, case.Lq, case.d
        nQB, nKB = Lq // 128, case.Lkv // case.kb
        gout = case.out.float().cpu().numpy().reshape(B * H, Lq, d)
        # the same forward with fp32 output (untimed): the kernel's error
        # without the final rounding to bf16, which alone is up to half a bf16
        # ulp (3.9e-3 at |o| in [1, 2))
        out32 = torch.empty(case.out.shape, dtype=torch.float32, device="cuda")
        case.fwd(out_dtype=torch.float32, out=out32)
        torch.cuda.synchronize()
        gout32 = out32.cpu().numpy().reshape(B * H, Lq, d)
        del out32
        mism = int(((bmap != cb["map"]) & (cb["tie"] == 0)).sum())
        errs, errs32 = [], []
        gm, om = bmap.reshape(B * H, nQB, nKB), cb["map"].reshape(B * H, nQB, nKB)
        for e, sid in enumerate(cb["sel"]):
            bh, i = divmod(int(sid), nQB)
            if (gm[bh, i] != om[bh, i]).any():
                continue
            r1 = min(128, max(0, wl.lq_valid - i * 128))
            errs.append(np.abs(gout[bh, i * 128:i * 128 + r1] - cb["out"][e, :r1]).reshape(-1))
            errs32.append(np.abs(gout32[bh, i * 128:i * 128 + r1] - cb["out"][e, :r1]).reshape(-1))
        err = np.concatenate(errs) if errs else np.zeros(1)
        err32 = np.concatenate(errs32) if errs32 else np.zeros(1)
        res["parity_sample"] = {"map_mismatches_outside_ties": mism, "ties": int(cb["tie"].sum()),
                                "max_abs": float(err.max()), "mean_abs": float(err.mean()), "out_dtype": "bf16",
                                "fp32_out": {"max_abs": float(err32.max()), "mean_abs": float(err32.mean())}}
    print(json.dumps(res), flush=True)
    del case
    torch.cuda.empty_cache()


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


def _probe_lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_int8_amd", "libsa_probe.so"))
    lib.sa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p]
    lib.sa_probe_bandwidth.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return lib


MFMA_PROBE_NAMES = {0: "int8_mfma_TOPS", 1: "bf16_mfma_TFLOPS", 2: "mixed_50_50_TOPS"}


def probe_mfma(torch, lib, mode, warmup=1, reps=3):
    """Sustained matrix-core rate of this GPU on random operands, in TOP/s:
    mode 0 int8 32x32x32, 1 bf16 32x32x16, 2 the forward's 50/50 mix (two int8
    and four bf16 MFMAs per iteration, interleaved).  Median of `reps` runs."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    g = torch.Generator().manual_seed(7)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (64 * 256,), dtype=torch.int64, generator=g).to(torch.int32).cuda()
    blocks = 256 * 8                       # 8 workgroups of 4 waves per CU: 8 waves per SIMD
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    iters = 4096
    # ops per MFMA: int8 32x32x32 = 2*32768, bf16 32x32x16 = 2*16384
    per_wave = {0: iters * 4 * 65536, 1: iters * 4 * 32768, 2: iters * (2 * 65536 + 4 * 32768)}[mode]
    ts = []
    for rep in range(reps + warmup):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert lib.sa_probe_mfma(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(sink.data_ptr()), mode, iters,
                                 blocks, sp) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        if rep >= warmup:
            ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    return per_wave * blocks * 4 / (ms * 1e-3) / 1e12, ms


def bench_peaks(args):
    """Matrix-core throughput (int8, bf16 and the forward's 50/50 mix, on
    random operands) and HBM read / write / copy bandwidth, measured with the
    probe kernels of libsa_probe.so."""
    import torch
    lib = _probe_lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(256 * 8 * 256, dtype=torch.int32, device="cuda")
    res = {"metric": "MI355X measured ceilings (probe kernels)", "unit": "TOP/s | GB/s", "n_gpus": 1}
    for mode in (0, 1, 2):
        tops, ms = probe_mfma(torch, lib, mode, warmup=args.warmup)
        nm = MFMA_PROBE_NAMES[mode]
        res[nm] = round(tops, 1)
        log(f"[peaks] {nm}: {res[nm]} ({ms:.3f} ms)")
    nbytes = 2 << 30
    x = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    y = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for kind, nm, mult in ((0, "hbm_read_GBps", 1), (1, "hbm_write_GBps", 1), (2, "hbm_copy_GBps", 2)):
        ts = []
        for rep in range(3 + args.warmup):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert lib.sa_probe_bandwidth(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), nbytes, kind,
                                          256 * 16, ctypes.c_void_p(sink.data_ptr()), sp) == 0
            e1.record(stream)
            torch.cuda.synchronize()
            if rep >= args.warmup:
                ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        res[nm] = round(nbytes * mult / (ms * 1e-3) / 1e9, 1)
        log(f"[peaks] {nm}: {res[nm]} ({ms:.3f} ms for {nbytes >> 20} MiB)")
    # torch's own copy and fill kernels on the same buffers, for comparison
    for nm, fn, mult in (("torch_copy_GBps", lambda: y.copy_(x), 2), ("torch_fill_GBps", lambda: y.fill_(5), 1)):
        ts = []
        for rep in range(3 + args.warmup):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if rep >= args.warmup:
                ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        res[nm] = round(nbytes * mult / (ms * 1e-3) / 1e9, 1)
        log(f"[peaks] {nm}: {res[nm]} ({ms:.3f} ms)")
    m8, mb = res["int8_mfma_TOPS"], res["bf16_mfma_TFLOPS"]
    res["mixed_harmonic_TOPS"] = round(1.0 / (0.5 / m8 + 0.5 / mb), 1)
    res["datasheet"] = {"int8_TOPS": PEAK_INT8, "bf16_TFLOPS": PEAK_BF16, "hbm_GBps": PEAK_HBM,
                        "mixed_harmonic_TOPS": round(1.0 / (0.5 / PEAK_INT8 + 0.5 / PEAK_BF16), 1)}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="3",
                    help="workload 1..5 (3 is the measured one; the others are the parity workloads), 'all' (1..5), "
                         "or 'seg' (the segmented key layout of the reference-conditioned video recipe)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-stride", type=int, default=0,
                    help="oracle forward on every n-th query block (0: a per-workload default)")
    ap.add_argument("--heads", type=int, default=40, help="heads of workload 3 (40 for the measured workload)")
    ap.add_argument("--rule", choices=["threshold", "topk"], default="threshold",
                    help="routing rule for the routed workloads: Sol threshold (the measured workload) or fixed "
                         "sparsity")
    ap.add_argument("--sparsity", type=float, default=0.75, help="pruned fraction for --rule topk")
    ap.add_argument("--qk-float", action="store_true",
                    help="exact tiles on the floating path (bf16 QK^T) instead of INT8 (same map and centroids)")
    ap.add_argument("--cache-append", action="store_true",
                    help="measure the streaming INT8 K/V cache append instead (FlashVSR-like: H=12, frames of "
                         "2048 rows, a ring of four frames)")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the matrix-core and HBM ceilings with the probe kernels instead")
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
    if args.peaks:
        bench_peaks(args)
        return
    if args.cache_append:
        bench_cache_append(args, sa, W)
        return
    configs = ([1, 2, 3, 4, 5] if args.config == "all" else [SEG] if args.config == "seg"
               else [int(args.config)])
    for n in configs:
        run_case(n, args, sa, W, torch)


if __name__ == "__main__":
    main()
