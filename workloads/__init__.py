"""Seeded synthetic inputs for the block-sparse INT8 video attention path.

This module draws random tensors and builds the static block patterns that the
workloads use.  It holds none of the attention method's arithmetic: no
quantization, no routing, no softmax.  Both the HIP path and the CPU oracle take
their inputs from here, and neither imports the other.

Every generator draws from ``numpy.random.default_rng(seed)`` (PCG64) in the
order documented on each function, produces float32 values and rounds them to
bfloat16 (round to nearest, ties to even).  bfloat16 tensors are returned as
``uint16`` arrays holding the raw bit patterns, shaped ``[B, H, L, d]``.

The workloads follow the shapes of the five pages' scenarios:

* tiny Sol routing (1x64 centroids),
* FlashVSR LCSA over an INT8 sliding K/V cache (FlashVSR Sparge Attention,
  "How it works"; FlashVSR Kitchen Sparse Attention, opening section),
* a Wan-14B-like long video sequence (Configure Sol Sparse Attention,
  opening section and "How it works"),
* Sol 2x32 with a dense-exempt conditioning prefix (Configure Sol Sparse
  Attention, "The inputs that matter"; Ref2VA VSA, the two-stage attention
  patch section),
* H3 static virtual KV in residual mode (Configure H3 Static Virtual KV,
  mode list).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DROP, EXACT, CENTROID = 0, 1, 2


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One attention call's inputs (host arrays) and its routing settings."""

    name: str
    B: int
    H: int
    Lq: int
    Lkv: int
    d: int
    lq_valid: int
    lkv_valid: int
    q: np.ndarray                      # bf16 bits [B,H,Lq,d]
    k: np.ndarray                      # bf16 bits [B,H,Lkv_phys,d] (physical K for virtual KV)
    v: np.ndarray                      # bf16 bits [B,H,Lv,d]
    threshold: float = 1.0
    rule: int = 0                      # 0: threshold rule; 1: fixed sparsity (top-k of the candidates)
    sparsity: float = 0.0              # fraction of candidates pruned under the fixed-sparsity rule
    centroids_per_block: int = 1
    prefix_tokens: int = 0
    segments: Optional[np.ndarray] = None      # int32 [n, 3] key layout: start, rows, routed (replaces the prefix)
    qk_float: bool = False             # exact tiles on the bf16 Q/K (floating QK path) instead of INT8
    kblock: int = 64
    k_scale_rows: int = 64
    v_int8: bool = False               # V handed over as an INT8 cache (quantized per v_scale_rows)
    v_scale_rows: int = 128
    explicit_map: Optional[np.ndarray] = None   # uint8 [B,H,nQB,Lkv/map_kblock]
    map_kblock: int = 64
    # virtual KV (K/V gathered from physical slices)
    virtual: bool = False
    rows_per_slice: int = 0
    n_phys: int = 0
    src_map: Optional[np.ndarray] = None        # int32 [n_logical]
    rope_cos: Optional[np.ndarray] = None       # float32 [n_logical, d_rot/2]
    rope_sin: Optional[np.ndarray] = None
    rot_offset: int = 0
    d_rot: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def dense_equiv_ops(self) -> float:
        return 4.0 * self.B * self.H * self.Lq * self.Lkv * self.d


def iid_normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal float32 draws in C order, rounded to bfloat16."""
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def framed_lowrank_bf16(rng: np.random.Generator, H: int, frame_len: int, n_frames: int,
                        d: int, rank: int = 8, rho: float = 0.5,
                        shared: Optional[tuple] = None):
    """Per-frame low-rank correlated tokens with unit variance per element.

    For head h and frame f a basis ``Bf`` (rank x d, entries N(0, 1/rank)) and a
    frame mean ``mf`` (N(0, I_rank)) are drawn, unless ``shared`` passes them in
    (Q and K share them).  Token t of frame f is
    ``sqrt(1-rho) z + sqrt(rho/2) (mf + n_t) Bf`` with ``z ~ N(0, I_d)`` and
    ``n_t ~ N(0, I_rank)``.  Draw order: (Bf, mf) if not shared, then z for all
    tokens [H, F*frame_len, d], then n for all tokens [H, F*frame_len, rank].
    Returns (bf16 bits [H, F*frame_len, d], (Bf, mf)).
    """
    if shared is None:
        basis = rng.standard_normal((H, n_frames, rank, d), dtype=np.float32) / np.float32(math.sqrt(rank))
        mean = rng.standard_normal((H, n_frames, rank), dtype=np.float32)
    else:
        basis, mean = shared
    L = n_frames * frame_len
    z = rng.standard_normal((H, L, d), dtype=np.float32)
    n = rng.standard_normal((H, L, rank), dtype=np.float32)
    coef = (n.reshape(H, n_frames, frame_len, rank) + mean[:, :, None, :]) * np.float32(math.sqrt(rho / 2.0))
    low = np.einsum("hftr,hfrd->hftd", coef, basis, optimize=True).reshape(H, L, d)
    x = np.float32(math.sqrt(1.0 - rho)) * z + low
    return bf16_bits(x.astype(np.float32)), (basis, mean)


def lcsa_map(B: int, H: int, n_frames: int, blocks_per_frame: int,
             frame_back: int = 1, radius: int = 2) -> np.ndarray:
    """Local-causal block pattern on 128x128 logical blocks.

    Query block (t, b) (frame t, in-frame block index b) attends key block
    (t', b') when ``t - frame_back <= t' <= t`` and ``|b' - b| <= radius``; every
    other block is dropped.  FlashVSR Sparge Attention, opening section and
    "How it works" (logical 128-query x 128-key blocks).
    """
    n = n_frames * blocks_per_frame
    m = np.zeros((n, n), dtype=np.uint8)
    for qi in range(n):
        t, b = divmod(qi, blocks_per_frame)
        for kj in range(n):
            t2, b2 = divmod(kj, blocks_per_frame)
            if t - frame_back <= t2 <= t and abs(b2 - b) <= radius:
                m[qi, kj] = EXACT
    return np.broadcast_to(m, (B, H, n, n)).copy()


def forced_residual_map(B: int, H: int, n_qblocks: int, n_kblocks: int, n_exact_kblocks: int) -> np.ndarray:
    """Virtual-KV residual pattern: the first ``n_exact_kblocks`` key blocks (the
    real slices) exact, all later ones as centroids.  Configure H3 Static
    Virtual KV, mode list ("residual")."""
    m = np.full((B, H, n_qblocks, n_kblocks), CENTROID, dtype=np.uint8)
    m[..., :n_exact_kblocks] = EXACT
    return m


def rope_tables(n_logical: int, d_rot: int, base: float = 10000.0):
    """Temporal rotary phases for logical slice l: angle l * base**(-2k/d_rot)
    for pair k.  Built in float64, handed over as float32 [n_logical, d_rot/2]."""
    k = np.arange(d_rot // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d_rot)
    ang = np.arange(n_logical, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ---------------------------------------------------------------------------
# The five workloads.  ``scale`` shrinks heads / frames for fast parity runs
# while keeping every structural feature (ragged tails, prefix, frames).
# ---------------------------------------------------------------------------

def tiny_sol(seed: int = 1, H: int = 2, L: int = 1024, d: int = 64, valid: Optional[int] = None,
             threshold: float = 1.0, centroids_per_block: int = 1) -> Workload:
    """i.i.d. N(0,1) Q, K, V (drawn in that order), Sol routing, no prefix."""
    rng = np.random.default_rng(seed)
    q = iid_normal_bf16(rng, (1, H, L, d))
    k = iid_normal_bf16(rng, (1, H, L, d))
    v = iid_normal_bf16(rng, (1, H, L, d))
    valid = L if valid is None else valid
    return Workload("tiny_sol_1x64", 1, H, L, L, d, valid, valid, q, k, v, threshold=threshold,
                    centroids_per_block=centroids_per_block)


def flashvsr_lcsa(seed: int = 2, H: int = 12, n_frames: int = 4, frame_tokens: int = 32 * 64,
                  d: int = 128) -> Workload:
    """Q, K, V i.i.d. N(0,1) (that order); K and V are handed to the path as an
    INT8 cache with one scale per 128 rows; LCSA pattern over 128x128 blocks."""
    rng = np.random.default_rng(seed)
    L = n_frames * frame_tokens
    q = iid_normal_bf16(rng, (1, H, L, d))
    k = iid_normal_bf16(rng, (1, H, L, d))
    v = iid_normal_bf16(rng, (1, H, L, d))
    bpf = frame_tokens // 128
    emap = lcsa_map(1, H, n_frames, bpf)
    return Workload("flashvsr_lcsa", 1, H, L, L, d, L, L, q, k, v, threshold=float("nan"),
                    centroids_per_block=0, kblock=128, k_scale_rows=128, v_int8=True, v_scale_rows=128,
                    explicit_map=emap, map_kblock=128)


def wan_like(seed: int = 3, H: int = 40, n_frames: int = 21, frame_tokens: int = 30 * 52,
             d: int = 128, pad_to: int = 128, threshold: float = 1.0) -> Workload:
    """Per-frame low-rank correlated Q/K (shared frame factors) and V (own
    factors), zero padding rows after the last frame up to a multiple of
    ``pad_to``.  Draw order: Q/K frame factors, Q tokens, K tokens, V factors,
    V tokens (see ``framed_lowrank_bf16``)."""
    rng = np.random.default_rng(seed)
    valid = n_frames * frame_tokens
    L = -(-valid // pad_to) * pad_to
    qv, shared = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d)
    kv, _ = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d, shared=shared)
    vv, _ = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d)

    def pad(x):
        out = np.zeros((1, H, L, d), dtype=np.uint16)
        out[0, :, :valid] = x
        return out

    return Workload("wan14b_like_sol_1x64", 1, H, L, L, d, valid, valid, pad(qv), pad(kv), pad(vv),
                    threshold=threshold)


def sol_prefix(seed: int = 4, H: int = 24, prefix: int = 1024, n_frames: int = 8,
               frame_tokens: int = 84 * 48, d: int = 128, threshold: float = 1.0) -> Workload:
    """A 1024-token conditioning prefix of i.i.d. N(0,1) tokens followed by
    video frames built like ``wan_like``.  Draw order: prefix Q, K, V, then the
    video part in ``wan_like``'s order."""
    rng = np.random.default_rng(seed)
    pq = iid_normal_bf16(rng, (H, prefix, d))
    pk = iid_normal_bf16(rng, (H, prefix, d))
    pv = iid_normal_bf16(rng, (H, prefix, d))
    qv, shared = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d)
    kv, _ = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d, shared=shared)
    vv, _ = framed_lowrank_bf16(rng, H, frame_tokens, n_frames, d)
    L = prefix + n_frames * frame_tokens
    cat = lambda a, b: np.concatenate([a, b], axis=1)[None]
    return Workload("sol_2x32_prefix", 1, H, L, L, d, L, L, cat(pq, qv), cat(pk, kv), cat(pv, vv),
                    threshold=threshold, centroids_per_block=2, prefix_tokens=prefix)


def virtual_kv_residual(seed: int = 5, H: int = 24, rows_per_slice: int = 2048, n_phys: int = 2,
                        n_logical: int = 7, d: int = 128, d_rot: int = 44) -> Workload:
    """Q, physical K, physical V i.i.d. N(0,1) (that order), then the source
    map: logical slices 0 and 1 read physical slices 0 and 1; slices 2..6 draw
    their physical slice with ``rng.integers(0, n_phys, n_logical - 2)``.
    Rotary tables per ``rope_tables``; the real slices' key blocks exact, the
    virtual ones as two 32-row centroids per block."""
    rng = np.random.default_rng(seed)
    Lq = n_phys * rows_per_slice
    q = iid_normal_bf16(rng, (1, H, Lq, d))
    k = iid_normal_bf16(rng, (1, H, n_phys * rows_per_slice, d))
    v = iid_normal_bf16(rng, (1, H, n_phys * rows_per_slice, d))
    src = np.concatenate([np.arange(n_phys), rng.integers(0, n_phys, n_logical - n_phys)]).astype(np.int32)
    cos, sin = rope_tables(n_logical, d_rot)
    Lkv = n_logical * rows_per_slice
    emap = forced_residual_map(1, H, Lq // 128, Lkv // 64, n_phys * rows_per_slice // 64)
    return Workload("virtual_kv_residual", 1, H, Lq, Lkv, d, Lq, Lkv, q, k, v, threshold=float("nan"),
                    centroids_per_block=2, kblock=64, k_scale_rows=64, explicit_map=emap, map_kblock=64,
                    virtual=True, rows_per_slice=rows_per_slice, n_phys=n_phys, src_map=src,
                    rope_cos=cos, rope_sin=sin, rot_offset=0, d_rot=d_rot)


def ref2va_segments(seed: int = 6, H: int = 24, text: int = 77, ref_image: int = 30 * 52, ref_audio: int = 250,
                    ref_video_frames: int = 2, video_frames: int = 8, frame_tokens: int = 30 * 52, d: int = 128,
                    kblock: int = 64, sparse_reference_video: bool = True, threshold: float = 1.0,
                    centroids_per_block: int = 1) -> Workload:
    """Reference-conditioned video self-attention over a segmented key layout
    (Ref2VA VSA, two-stage attention patch; Configure Sol Sparse Attention, "The
    inputs that matter"): prompt text, a reference image and reference audio
    (dense), a reference video clip (routed when ``sparse_reference_video``),
    then the generated video (routed).  Each segment starts on a key-block
    boundary; the rows between its end and the next start are zero padding, as
    are the rows after the last segment up to a multiple of 128.
    Draw order: text, reference image, reference audio (each Q, K, V i.i.d.
    N(0,1)), then all video frames (reference clip first) like ``wan_like``."""
    rng = np.random.default_rng(seed)
    dense = []
    for rows in (text, ref_image, ref_audio):
        dense.append(tuple(iid_normal_bf16(rng, (H, rows, d)) for _ in range(3)))
    nf = ref_video_frames + video_frames
    qv, shared = framed_lowrank_bf16(rng, H, frame_tokens, nf, d)
    kv, _ = framed_lowrank_bf16(rng, H, frame_tokens, nf, d, shared=shared)
    vv, _ = framed_lowrank_bf16(rng, H, frame_tokens, nf, d)
    cut = ref_video_frames * frame_tokens
    parts = dense + [(qv[:, :cut], kv[:, :cut], vv[:, :cut]), (qv[:, cut:], kv[:, cut:], vv[:, cut:])]
    routed = [0, 0, 0, 1 if sparse_reference_video else 0, 1]
    segs, cursor = [], 0
    for (pq, _, _), rt in zip(parts, routed):
        rows = pq.shape[1]
        if rows == 0:
            continue
        segs.append((cursor, rows, rt))
        cursor += -(-rows // kblock) * kblock
    L = -(-cursor // 128) * 128
    q = np.zeros((1, H, L, d), dtype=np.uint16)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    parts = [p for p in parts if p[0].shape[1] > 0]
    for (start, rows, _), (pq, pk, pv) in zip(segs, parts):
        q[0, :, start:start + rows] = pq
        k[0, :, start:start + rows] = pk
        v[0, :, start:start + rows] = pv
    end = segs[-1][0] + segs[-1][1]
    return Workload("ref2va_segments", 1, H, L, L, d, end, end, q, k, v, threshold=threshold,
                    centroids_per_block=centroids_per_block, kblock=kblock, k_scale_rows=kblock,
                    segments=np.array(segs, dtype=np.int32))


CONFIG_NAMES = {
    1: "tiny Sol 1x64 (H=2, d=64, L=1024)",
    2: "FlashVSR LCSA over an INT8 cache (H=12, d=128, L=8192)",
    3: "Wan-14B-like Sol 1x64 (H=40, d=128, L=32768, 32760 valid, thr=1.0)",
    4: "Sol 2x32 with 1024-token dense prefix (H=24, d=128, L=33280)",
    5: "virtual KV residual (H=24, d=128, Lq=4096, Lkv=14336 logical)",
}


def config(n: int, small: bool = False) -> Workload:
    """Full-size workload ``n`` (1..5); ``small=True`` gives a reduced version
    with the same structure (several tiles, ragged tails) for fast checks."""
    if n == 1:
        return tiny_sol()
    if n == 2:
        return flashvsr_lcsa(H=2, n_frames=3, frame_tokens=8 * 128) if small else flashvsr_lcsa()
    if n == 3:
        return wan_like(H=2, n_frames=5, frame_tokens=30 * 26) if small else wan_like()
    if n == 4:
        return sol_prefix(H=2, n_frames=3, frame_tokens=32 * 44) if small else sol_prefix()
    if n == 5:
        return virtual_kv_residual(H=2, rows_per_slice=512) if small else virtual_kv_residual()
    raise ValueError(f"unknown workload {n}")
