"""Python binding of libsparse_attn (block-sparse INT8 video attention on MI355X).

Argument marshalling only: every step of the computation runs in the library's
gfx950 HIP kernels.  PyTorch supplies device memory and the current HIP stream.
The entry points keep the C names:

    quantize_qk_int8, sparse_attn_route, sparse_attn_fwd, sparse_attn_fwd_float,
    gather_virtual_kv, kv_cache_append_int8

plus ``sparse_attention`` which chains quantize -> route -> fwd.

Loading (FlashVSR Kitchen Sparse Attention, "When it bites"): the library is
looked up in ``$SA_LIB`` and next to this file; if it is missing a
FileNotFoundError lists every place searched, a library built for another ABI
version is refused, and a non-gfx950 device is rejected.  There is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

ABI_VERSION = 7
SA_OK, SA_E_NULL, SA_E_SHAPE, SA_E_ALIGN, SA_E_VALUE, SA_E_UNSUPPORTED, SA_E_DEVICE, SA_E_LAUNCH, SA_E_WORKSPACE = range(9)
SA_DROP, SA_EXACT, SA_CENTROID = 0, 1, 2
SA_BF16, SA_INT8, SA_F32 = 0, 1, 2
SA_RULE_THRESHOLD, SA_RULE_TOPK = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
LIB_NAME = "libsparse_attn.so"


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[sa status {code}] {message}")
        self.code = code


class sa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "Lq", "Lkv", "d", "lq_valid", "lkv_valid", "Lv")]


class sa_segment(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("start", "rows", "routed")]


class sa_route_params(ctypes.Structure):
    _fields_ = [("threshold", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("centroids_per_block", "prefix_tokens", "kblock", "k_scale_rows",
                                      "v_scale_rows", "map_kblock", "rule")] + [
        ("sparsity", ctypes.c_float), ("n_segments", ctypes.c_int32),
        ("segments_host", ctypes.POINTER(sa_segment))]


def search_paths():
    paths = []
    env = os.environ.get("SA_LIB")
    if env:
        paths.append(env if env.endswith(".so") else os.path.join(env, LIB_NAME))
    paths.append(os.path.join(_HERE, LIB_NAME))
    return paths


def load(path: Optional[str] = None):
    """Load libsparse_attn.so (once) and check its ABI version."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    candidates = [path] if path else search_paths()
    found = next((p for p in candidates if p and os.path.isfile(p)), None)
    if found is None:
        raise FileNotFoundError(
            "libsparse_attn.so not found; searched: " + ", ".join(candidates) +
            " (build it with __graft_entry__.build() or block_sparse_int8_amd/_build.py)")
    lib = ctypes.CDLL(found)
    lib.sa_abi_version.restype = ctypes.c_int32
    got = lib.sa_abi_version()
    if got != ABI_VERSION:
        raise ImportError(f"{found} has ABI version {got}, this binding needs {ABI_VERSION}")
    lib.sa_last_error.restype = ctypes.c_char_p
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    P = ctypes.POINTER
    lib.sa_device_check.argtypes = [i32]
    lib.sa_device_check.restype = i32
    lib.quantize_qk_int8.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp]
    lib.quantize_qk_int8.restype = i32
    lib.sparse_attn_route_workspace_size.argtypes = [P(sa_dims), P(sa_route_params), i32]
    lib.sparse_attn_route_workspace_size.restype = ctypes.c_size_t
    lib.sparse_attn_route.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, P(sa_dims), P(sa_route_params), vp, vp,
                                      vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sparse_attn_route.restype = i32
    lib.sparse_attn_route_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, P(sa_dims), P(sa_route_params),
                                              vp, vp, vp, vp, vp, vp, vp]
    lib.sparse_attn_route_noalloc.restype = i32
    lib.sparse_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, P(sa_dims), P(sa_route_params), vp, vp, vp, vp,
                                    f32, vp, i32, vp, vp]
    lib.sparse_attn_fwd.restype = i32
    lib.gather_virtual_kv.argtypes = [vp, i32, i32, i32, i32, i32, vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.gather_virtual_kv.restype = i32
    lib.kv_cache_append_int8.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, vp, i32, i32, vp]
    lib.kv_cache_append_int8.restype = i32
    lib.sparse_attn_fwd_float.argtypes = [vp, vp, vp, vp, P(sa_dims), P(sa_route_params), vp, vp, vp, vp, f32, vp,
                                          i32, vp, vp]
    lib.sparse_attn_fwd_float.restype = i32
    if path is None:
        _LIB = lib
    return lib


def library_path() -> str:
    return load()._name


def _check(rc: int):
    if rc != SA_OK:
        raise SparseAttnError(rc, load().sa_last_error().decode())


def device_check(device: int = 0):
    _check(load().sa_device_check(device))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _keep_for(stream, *tensors):
    """Tensors allocated here (on torch's current stream) that kernels queued on
    another ``stream`` use: record that stream on them, so the caching
    allocator does not hand their memory out again before those kernels are
    done, even when the Python objects are released first."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
        stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_qk_int8(x: torch.Tensor, valid_len: Optional[int] = None, rows_per_block: int = 128,
                     out: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None, stream=None,
                     col_sums=False, sum_rows: Optional[int] = None):
    """bf16 [B,H,L,d] (any strides over B, H, L) -> (int8 [B,H,L,d], fp32 [B,H,L/R]).
    ``col_sums`` True (or an int16 [B,H,L/sum_rows,d] tensor) also writes the
    codes' column sums per chunk of ``sum_rows`` rows (32 or rows_per_block;
    default: rows_per_block for 128-row blocks, the route's Q sums, else 32,
    the route's K sums) and returns them as a third element."""
    if x.dim() != 4:
        raise ValueError("x must be [B,H,L,d]")
    _need(x, "x", torch.bfloat16, contiguous=False)
    B, H, L, d = x.shape
    if x.stride(3) != 1:
        raise ValueError("x must have a contiguous channel dimension")
    valid_len = L if valid_len is None else valid_len
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((B, H, L // rows_per_block if rows_per_block else 0), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.int8, (B, H, L, d))
    _need(scale, "scale", torch.float32, (B, H, L // rows_per_block))
    sums = None
    if sum_rows is None:
        sum_rows = 128 if rows_per_block == 128 else 32
    if col_sums is not False and col_sums is not None:
        sums = col_sums if isinstance(col_sums, torch.Tensor) else torch.empty(
            (B, H, L // sum_rows, d), dtype=torch.int16, device=x.device)
        _need(sums, "col_sums", torch.int16, (B, H, L // sum_rows, d))
    _check(load().quantize_qk_int8(_ptr(x), x.stride(0), x.stride(1), x.stride(2), B, H, L, d, valid_len,
                                   rows_per_block, _ptr(out), _ptr(scale), _ptr(sums), sum_rows, _stream(stream)))
    _keep_for(stream, out, scale, sums)
    return (out, scale) if sums is None else (out, scale, sums)


def kv_cache_append_int8(x: torch.Tensor, cache_q: torch.Tensor, cache_scale: torch.Tensor, first_slot: int,
                         valid_len: Optional[int] = None, rows_per_slab: int = 128, stream=None):
    """Quantize the bf16 chunk x [B,H,rows,d] per slab into ring slots
    (first_slot + s) % slots of cache_q int8 [B,H,slots*R,d] and cache_scale
    fp32 [B,H,slots], in place.  Returns the next free slot."""
    if x.dim() != 4:
        raise ValueError("x must be [B,H,rows,d]")
    _need(x, "x", torch.bfloat16, contiguous=False)
    B, H, rows, d = x.shape
    if x.stride(3) != 1:
        raise ValueError("x must have a contiguous channel dimension")
    if cache_scale.dim() != 3:
        raise ValueError("cache_scale must be [B,H,slots]")
    slots = cache_scale.shape[2]
    _need(cache_q, "cache_q", torch.int8, (B, H, slots * rows_per_slab, d))
    _need(cache_scale, "cache_scale", torch.float32, (B, H, slots))
    valid_len = rows if valid_len is None else valid_len
    _check(load().kv_cache_append_int8(_ptr(x), x.stride(0), x.stride(1), x.stride(2), B, H, rows, d, valid_len,
                                       rows_per_slab, _ptr(cache_q), _ptr(cache_scale), slots, first_slot,
                                       _stream(stream)))
    return (first_slot + rows // rows_per_slab) % slots


def _dims(B, H, Lq, Lkv, d, lq_valid, lkv_valid, Lv):
    return sa_dims(B, H, Lq, Lkv, d, lq_valid, lkv_valid, Lv)


def _params(threshold, G, prefix, kblock, k_scale_rows, v_scale_rows, map_kblock, rule=SA_RULE_THRESHOLD,
            sparsity=0.0, segments=None):
    """The parameter struct; ``segments`` is a sequence of (start, rows, routed).
    The struct keeps a reference to its segment array."""
    segs = [] if segments is None else [tuple(int(x) for x in g) for g in segments]
    arr = (sa_segment * max(1, len(segs)))(*[sa_segment(*g) for g in segs])
    prm = sa_route_params(float(threshold), G, prefix, kblock, k_scale_rows, v_scale_rows, map_kblock, int(rule),
                          float(sparsity), len(segs), ctypes.cast(arr, ctypes.POINTER(sa_segment)) if segs else None)
    prm._segments_keepalive = arr
    return prm


def sparse_attn_route(q8: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor, v: torch.Tensor, *,
                      lq_valid: Optional[int] = None, lkv_valid: Optional[int] = None,
                      v_scale: Optional[torch.Tensor] = None, v_block_src: Optional[torch.Tensor] = None,
                      threshold: float = 1.0, centroids_per_block: int = 1, prefix_tokens: int = 0,
                      kblock: int = 64, k_scale_rows: Optional[int] = None, v_scale_rows: int = 128,
                      explicit_map: Optional[torch.Tensor] = None, map_kblock: Optional[int] = None,
                      rule: int = SA_RULE_THRESHOLD, sparsity: float = 0.0, segments=None,
                      row_stats: bool = False, workspace: Optional[torch.Tensor] = None,
                      outputs: Optional[dict] = None, noalloc: bool = False,
                      q_sums: Optional[torch.Tensor] = None, k_sums: Optional[torch.Tensor] = None,
                      stream=None) -> dict:
    """Block map + centroids.  ``rule`` picks the threshold rule (``threshold``)
    or the fixed-sparsity rule (``sparsity``); ``segments`` ((start, rows,
    routed) triples) gives a segmented key layout in place of the prefix.
    Returns dict(map, k_centroid, v_centroid, count, row_stats) with the shapes
    of sparse_attn.h.  ``q_sums`` / ``k_sums``: the column sums quantize_qk_int8
    returned with q8 / k8 (the route then reads the sums, not the codes).
    ``noalloc`` calls sparse_attn_route_noalloc (library-owned
    workspace; pass every output in ``outputs`` for a call that allocates
    nothing)."""
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    Lv = v.shape[2]
    lq_valid = Lq if lq_valid is None else lq_valid
    lkv_valid = Lkv if lkv_valid is None else lkv_valid
    k_scale_rows = kblock if k_scale_rows is None else k_scale_rows
    map_kblock = kblock if map_kblock is None else map_kblock
    G = centroids_per_block
    _need(q8, "q8", torch.int8, (B, H, Lq, d))
    _need(k8, "k8", torch.int8, (B, H, Lkv, d))
    _need(k_scale, "k_scale", torch.float32, (B, H, Lkv // k_scale_rows))
    v_dtype = SA_INT8 if v.dtype == torch.int8 else SA_BF16
    _need(v, "v", torch.int8 if v_dtype == SA_INT8 else torch.bfloat16, (B, H, Lv, d))
    if v_dtype == SA_INT8:
        _need(v_scale, "v_scale", torch.float32, (B, H, Lv // v_scale_rows))
    if v_block_src is not None:
        _need(v_block_src, "v_block_src", torch.int32, (Lkv // 64,))
    if q_sums is not None:
        _need(q_sums, "q_sums", torch.int16, (B, H, Lq // 128, d))
    if k_sums is not None:
        _need(k_sums, "k_sums", torch.int16, (B, H, Lkv // 32, d))
    nQB, nKB = Lq // 128, Lkv // kblock
    if explicit_map is not None:
        _need(explicit_map, "explicit_map", torch.uint8, (B, H, nQB, Lkv // map_kblock))
    dims = _dims(B, H, Lq, Lkv, d, lq_valid, lkv_valid, Lv)
    prm = _params(threshold, G, prefix_tokens, kblock, k_scale_rows, v_scale_rows, map_kblock, rule, sparsity,
                  segments)
    lib = load()
    outputs = {} if outputs is None else outputs
    dev = q8.device
    bmap = outputs.get("map")
    if bmap is None:
        bmap = torch.empty((B, H, nQB, nKB), dtype=torch.uint8, device=dev)
    kc = vc = cnt = None
    if G > 0:
        kc = outputs.get("k_centroid")
        vc = outputs.get("v_centroid")
        cnt = outputs.get("count")
        if kc is None:
            kc = torch.empty((B, H, nKB, G, d), dtype=torch.float32, device=dev)
            vc = torch.empty((B, H, nKB, G, d), dtype=torch.float32, device=dev)
            cnt = torch.empty((B, H, nKB, G), dtype=torch.float32, device=dev)
    stats = outputs.get("row_stats")
    if stats is None and row_stats:
        stats = torch.empty((B, H, nQB, 2), dtype=torch.float64, device=dev)
    if stats is not None:
        _need(stats, "row_stats", torch.float64, (B, H, nQB, 2))
    if noalloc:
        _check(lib.sparse_attn_route_noalloc(_ptr(q8), _ptr(k8), _ptr(k_scale), _ptr(v), v_dtype, _ptr(v_scale),
                                             _ptr(v_block_src), _ptr(q_sums), _ptr(k_sums), ctypes.byref(dims),
                                             ctypes.byref(prm),
                                             _ptr(explicit_map), _ptr(bmap), _ptr(kc), _ptr(vc), _ptr(cnt),
                                             _ptr(stats), _stream(stream)))
        _keep_for(stream, bmap, kc, vc, cnt, stats)
        return dict(map=bmap, k_centroid=kc, v_centroid=vc, count=cnt, row_stats=stats, workspace=None)
    ws_bytes = lib.sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm),
                                                    1 if explicit_map is not None else 0)
    if workspace is None and ws_bytes:
        workspace = torch.empty((ws_bytes + 256,), dtype=torch.uint8, device=dev)
    ws_ptr, ws_avail = None, 0
    if workspace is not None:
        base = workspace.data_ptr()
        off = (-base) % 256
        ws_ptr = ctypes.c_void_p(base + off)
        ws_avail = workspace.numel() - off
    _check(lib.sparse_attn_route(_ptr(q8), _ptr(k8), _ptr(k_scale), _ptr(v), v_dtype, _ptr(v_scale),
                                 _ptr(v_block_src), _ptr(q_sums), _ptr(k_sums), ctypes.byref(dims),
                                 ctypes.byref(prm), _ptr(explicit_map),
                                 _ptr(bmap), _ptr(kc), _ptr(vc), _ptr(cnt), _ptr(stats), ws_ptr, ws_avail,
                                 _stream(stream)))
    _keep_for(stream, bmap, kc, vc, cnt, stats, workspace)
    return dict(map=bmap, k_centroid=kc, v_centroid=vc, count=cnt, row_stats=stats, workspace=workspace)


def sparse_attn_route_noalloc(q8: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor, v: torch.Tensor,
                              **kw) -> dict:
    """sparse_attn_route on the library-owned workspace (no ``workspace``
    argument); see sparse_attn_route for the keywords."""
    kw.pop("workspace", None)
    return sparse_attn_route(q8, k8, k_scale, v, noalloc=True, **kw)


def sparse_attn_fwd(q8: torch.Tensor, q_scale: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor,
                    v: torch.Tensor, block_map: torch.Tensor, *, k_centroid=None, v_centroid=None, count=None,
                    lq_valid: Optional[int] = None, lkv_valid: Optional[int] = None,
                    v_scale: Optional[torch.Tensor] = None, v_block_src: Optional[torch.Tensor] = None,
                    centroids_per_block: int = 1, kblock: int = 64, k_scale_rows: Optional[int] = None,
                    v_scale_rows: int = 128, sm_scale: Optional[float] = None,
                    out_dtype: torch.dtype = torch.float32, return_lse: bool = False,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, segments=None,
                    stream=None):
    """Attention output [B,H,Lq,d] (and lse [B,H,Lq] when asked).  ``segments``
    must be the key layout the map was routed with."""
    B, H, Lq, d = q8.shape
    Lkv = k8.shape[2]
    Lv = v.shape[2]
    lq_valid = Lq if lq_valid is None else lq_valid
    lkv_valid = Lkv if lkv_valid is None else lkv_valid
    k_scale_rows = kblock if k_scale_rows is None else k_scale_rows
    G = centroids_per_block
    nQB, nKB = Lq // 128, Lkv // kblock
    _need(q8, "q8", torch.int8, (B, H, Lq, d))
    _need(q_scale, "q_scale", torch.float32, (B, H, nQB))
    _need(k8, "k8", torch.int8, (B, H, Lkv, d))
    _need(k_scale, "k_scale", torch.float32, (B, H, Lkv // k_scale_rows))
    v_dtype = SA_INT8 if v.dtype == torch.int8 else SA_BF16
    _need(v, "v", torch.int8 if v_dtype == SA_INT8 else torch.bfloat16, (B, H, Lv, d))
    if v_dtype == SA_INT8:
        _need(v_scale, "v_scale", torch.float32, (B, H, Lv // v_scale_rows))
    if v_block_src is not None:
        _need(v_block_src, "v_block_src", torch.int32, (Lkv // 64,))
    _need(block_map, "block_map", torch.uint8, (B, H, nQB, nKB))
    if G > 0:
        _need(k_centroid, "k_centroid", torch.float32, (B, H, nKB, G, d))
        _need(v_centroid, "v_centroid", torch.float32, (B, H, nKB, G, d))
        _need(count, "count", torch.float32, (B, H, nKB, G))
    odt = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[out_dtype]
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=out_dtype, device=q8.device)
    _need(out, "out", out_dtype, (B, H, Lq, d))
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, Lq))
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    dims = _dims(B, H, Lq, Lkv, d, lq_valid, lkv_valid, Lv)
    prm = _params(float("nan"), G, 0, kblock, k_scale_rows, v_scale_rows, kblock, segments=segments)
    _check(load().sparse_attn_fwd(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), v_dtype, _ptr(v_scale),
                                  _ptr(v_block_src), ctypes.byref(dims), ctypes.byref(prm), _ptr(block_map),
                                  _ptr(k_centroid), _ptr(v_centroid), _ptr(count), float(sm), _ptr(out), odt,
                                  _ptr(lse), _stream(stream)))
    _keep_for(stream, out, lse)
    return (out, lse) if return_lse else out


def sparse_attn_fwd_float(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_map: torch.Tensor, *,
                          k_centroid=None, v_centroid=None, count=None, lq_valid: Optional[int] = None,
                          lkv_valid: Optional[int] = None, v_block_src: Optional[torch.Tensor] = None,
                          centroids_per_block: int = 1, kblock: int = 64, sm_scale: Optional[float] = None,
                          out_dtype: torch.dtype = torch.float32, return_lse: bool = False,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, segments=None,
                          stream=None):
    """Forward with a floating QK^T on bf16 q [B,H,Lq,d], k [B,H,Lkv,d],
    v [B,H,Lv,d]; map and centroids from sparse_attn_route."""
    B, H, Lq, d = q.shape
    Lkv, Lv = k.shape[2], v.shape[2]
    lq_valid = Lq if lq_valid is None else lq_valid
    lkv_valid = Lkv if lkv_valid is None else lkv_valid
    G = centroids_per_block
    nQB, nKB = Lq // 128, Lkv // kblock
    _need(q, "q", torch.bfloat16, (B, H, Lq, d))
    _need(k, "k", torch.bfloat16, (B, H, Lkv, d))
    _need(v, "v", torch.bfloat16, (B, H, Lv, d))
    if v_block_src is not None:
        _need(v_block_src, "v_block_src", torch.int32, (Lkv // 64,))
    _need(block_map, "block_map", torch.uint8, (B, H, nQB, nKB))
    if G > 0:
        _need(k_centroid, "k_centroid", torch.float32, (B, H, nKB, G, d))
        _need(v_centroid, "v_centroid", torch.float32, (B, H, nKB, G, d))
        _need(count, "count", torch.float32, (B, H, nKB, G))
    odt = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[out_dtype]
    if out is None:
        out = torch.empty((B, H, Lq, d), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype, (B, H, Lq, d))
    if return_lse and lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, Lq))
    sm = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    dims = _dims(B, H, Lq, Lkv, d, lq_valid, lkv_valid, Lv)
    prm = _params(float("nan"), G, 0, kblock, kblock, 128, kblock, segments=segments)
    _check(load().sparse_attn_fwd_float(_ptr(q), _ptr(k), _ptr(v), _ptr(v_block_src), ctypes.byref(dims),
                                        ctypes.byref(prm), _ptr(block_map), _ptr(k_centroid), _ptr(v_centroid),
                                        _ptr(count), float(sm), _ptr(out), odt, _ptr(lse), _stream(stream)))
    _keep_for(stream, out, lse)
    return (out, lse) if return_lse else out


def gather_virtual_kv(k_phys: torch.Tensor, rows_per_slice: int, src_map: Sequence[int], rope_cos: torch.Tensor,
                      rope_sin: torch.Tensor, rot_offset: int = 0, k_rows_per_block: int = 64, stream=None):
    """Physical bf16 K [B,H,n_phys*S,d] -> (int8 logical K, fp32 scales, int32 V block table)."""
    _need(k_phys, "k_phys", torch.bfloat16)
    B, H, Lp, d = k_phys.shape
    S = rows_per_slice
    n_logical = len(src_map)
    _need(rope_cos, "rope_cos", torch.float32)
    _need(rope_sin, "rope_sin", torch.float32, tuple(rope_cos.shape))
    if rope_cos.dim() != 2 or rope_cos.shape[0] != n_logical:
        raise ValueError("rope tables must be [n_logical, d_rot/2]")
    d_rot = 2 * rope_cos.shape[1]
    src = (ctypes.c_int32 * n_logical)(*[int(s) for s in src_map])
    Ll = n_logical * S
    kq = torch.empty((B, H, Ll, d), dtype=torch.int8, device=k_phys.device)
    ks = torch.empty((B, H, Ll // k_rows_per_block), dtype=torch.float32, device=k_phys.device)
    vbs = torch.empty((Ll // 64,), dtype=torch.int32, device=k_phys.device)
    _check(load().gather_virtual_kv(_ptr(k_phys), B, H, S, Lp // S if S else 0, d, src, n_logical, _ptr(rope_cos),
                                    _ptr(rope_sin), rot_offset, d_rot, k_rows_per_block, _ptr(kq), _ptr(ks),
                                    _ptr(vbs), _stream(stream)))
    _keep_for(stream, kq, ks, vbs)
    return kq, ks, vbs


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, lq_valid=None, lkv_valid=None,
                     threshold: float = 1.0, centroids_per_block: int = 1, prefix_tokens: int = 0,
                     explicit_map: Optional[torch.Tensor] = None, map_kblock: Optional[int] = None,
                     rule: int = SA_RULE_THRESHOLD, sparsity: float = 0.0, segments=None, kblock: int = 64,
                     sm_scale: Optional[float] = None, out_dtype=torch.float32,
                     return_lse: bool = False, stream=None):
    """quantize_qk_int8(Q, 128 rows) -> quantize_qk_int8(K, kblock rows) ->
    sparse_attn_route -> sparse_attn_fwd, all on one stream.  q, k, v are bf16
    [B,H,L,d]; V stays bf16."""
    Lq, Lkv = q.shape[2], k.shape[2]
    lq_valid = Lq if lq_valid is None else lq_valid
    lkv_valid = Lkv if lkv_valid is None else lkv_valid
    q8, qs, qsum = quantize_qk_int8(q, lq_valid, 128, stream=stream, col_sums=True, sum_rows=128)
    k8, ks, ksum = quantize_qk_int8(k, lkv_valid, kblock, stream=stream, col_sums=True, sum_rows=32)
    r = sparse_attn_route(q8, k8, ks, v, q_sums=qsum, k_sums=ksum, lq_valid=lq_valid, lkv_valid=lkv_valid,
                          threshold=threshold,
                          centroids_per_block=centroids_per_block, prefix_tokens=prefix_tokens, kblock=kblock,
                          explicit_map=explicit_map, map_kblock=map_kblock, rule=rule, sparsity=sparsity,
                          segments=segments, stream=stream)
    res = sparse_attn_fwd(q8, qs, k8, ks, v, r["map"], k_centroid=r["k_centroid"], v_centroid=r["v_centroid"],
                          count=r["count"], lq_valid=lq_valid, lkv_valid=lkv_valid,
                          centroids_per_block=centroids_per_block, kblock=kblock, sm_scale=sm_scale,
                          out_dtype=out_dtype, return_lse=return_lse, segments=segments, stream=stream)
    return res, r["map"]
