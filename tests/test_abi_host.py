"""Host-only checks of the C ABI (no GPU needed, no kernel launched).

FlashVSR Kitchen Sparse Attention, "When it bites": a missing library fails at
once and lists where it looked; an incompatible ABI version fails fast;
unsupported devices are rejected outright.
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_int8_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("quantize_qk_int8", "sparse_attn_route", "sparse_attn_fwd", "gather_virtual_kv", "kv_cache_append_int8",
              "sparse_attn_fwd_float",
              "sa_abi_version", "sa_last_error", "sa_device_check", "sparse_attn_route_workspace_size"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sa.library_path())
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} declared in sparse_attn.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", sa.library_path()], capture_output=True, text=True).stdout
    for n in _declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_abi_version():
    assert sa.load().sa_abi_version() == sa.ABI_VERSION == 7


def test_missing_library_lists_search_paths(monkeypatch, tmp_path):
    monkeypatch.setenv("SA_LIB", str(tmp_path / "nowhere"))
    with pytest.raises(FileNotFoundError) as ei:
        sa.load(path=str(tmp_path / "nowhere" / "libsparse_attn.so"))
    assert "nowhere" in str(ei.value)
    paths = sa.search_paths()
    assert str(tmp_path / "nowhere" / "libsparse_attn.so") in paths


def test_wrong_abi_version_is_refused(tmp_path):
    src = tmp_path / "stub.c"
    src.write_text("int sa_abi_version(void) { return 99; }\n")
    so = tmp_path / "libsparse_attn.so"
    subprocess.run(["gcc", "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    with pytest.raises(ImportError, match="ABI version 99"):
        sa.load(path=str(so))


def _lib():
    return sa.load()


def _err():
    return _lib().sa_last_error().decode()


def test_quantize_validation_before_any_device_call():
    lib = _lib()
    p = ctypes.c_void_p(16)     # never dereferenced: validation fails first
    assert lib.quantize_qk_int8(None, 0, 0, 0, 1, 1, 128, 128, 128, 128, p, p, None, 32, None) == sa.SA_E_NULL
    assert lib.quantize_qk_int8(p, 0, 0, 128, 1, 1, 128, 96, 128, 128, p, p, None, 32, None) == sa.SA_E_SHAPE
    assert "d must be" in _err()
    assert lib.quantize_qk_int8(p, 0, 0, 128, 1, 1, 128, 128, 128, 32, p, p, None, 32, None) == sa.SA_E_VALUE
    assert lib.quantize_qk_int8(p, 0, 0, 128, 1, 1, 100, 128, 100, 64, p, p, None, 32, None) == sa.SA_E_SHAPE
    assert lib.quantize_qk_int8(p, 0, 0, 128, 1, 1, 128, 128, 129, 64, p, p, None, 32, None) == sa.SA_E_SHAPE
    assert lib.quantize_qk_int8(ctypes.c_void_p(8), 0, 0, 128, 1, 1, 128, 128, 128, 64, p, p, None, 32, None) == sa.SA_E_ALIGN
    assert lib.quantize_qk_int8(p, 0, 0, 100, 1, 1, 128, 128, 128, 64, p, p, None, 32, None) == sa.SA_E_ALIGN


def _dims(**kw):
    d = dict(B=1, H=1, Lq=256, Lkv=256, d=128, lq_valid=256, lkv_valid=256, Lv=256)
    d.update(kw)
    return sa.sa_dims(*[d[k] for k in ("B", "H", "Lq", "Lkv", "d", "lq_valid", "lkv_valid", "Lv")])


def _prm(**kw):
    d = dict(threshold=1.0, centroids_per_block=1, prefix_tokens=0, kblock=64, k_scale_rows=64, v_scale_rows=128,
             map_kblock=64, rule=sa.SA_RULE_THRESHOLD, sparsity=0.0, segments=None)
    d.update(kw)
    return sa._params(d["threshold"], *[d[k] for k in ("centroids_per_block", "prefix_tokens", "kblock",
                                                           "k_scale_rows", "v_scale_rows", "map_kblock",
                                                           "rule", "sparsity", "segments")])


def _route(dims, prm, em=None, ws=None, wsb=0, G_out=True):
    lib = _lib()
    p = ctypes.c_void_p(256)
    c = p if G_out else None
    return lib.sparse_attn_route(p, p, p, p, sa.SA_BF16, None, None, None, None, ctypes.byref(dims), ctypes.byref(prm),
                                 em, p,
                                 c, c, c, None, ws, wsb, None)


@pytest.mark.parametrize("dims_kw,prm_kw,code,msg", [
    (dict(d=96), {}, sa.SA_E_SHAPE, "d must be"),
    (dict(Lq=200), {}, sa.SA_E_SHAPE, "Lq must be"),
    (dict(lkv_valid=300), {}, sa.SA_E_SHAPE, "lkv_valid"),
    (dict(Lv=128), {}, sa.SA_E_SHAPE, "Lv"),
    ({}, dict(kblock=32), sa.SA_E_VALUE, "kblock"),
    ({}, dict(prefix_tokens=100), sa.SA_E_VALUE, "prefix"),
    ({}, dict(threshold=float("nan")), sa.SA_E_VALUE, "NaN"),
    ({}, dict(centroids_per_block=0), sa.SA_E_VALUE, "centroids"),
    ({}, dict(centroids_per_block=3), sa.SA_E_VALUE, "centroids"),
    ({}, dict(k_scale_rows=128), sa.SA_E_VALUE, "k_scale_rows == kblock"),
    ({}, dict(rule=2), sa.SA_E_VALUE, "rule must be"),
    ({}, dict(rule=sa.SA_RULE_TOPK, sparsity=1.5), sa.SA_E_VALUE, "sparsity"),
    ({}, dict(rule=sa.SA_RULE_TOPK, sparsity=-0.25), sa.SA_E_VALUE, "sparsity"),
    ({}, dict(rule=sa.SA_RULE_TOPK, sparsity=float("nan")), sa.SA_E_VALUE, "sparsity"),
    ({}, dict(rule=sa.SA_RULE_TOPK, sparsity=0.5, k_scale_rows=128), sa.SA_E_VALUE, "k_scale_rows == kblock"),
    ({}, dict(segments=[(0, 64, 0), (100, 64, 1)]), sa.SA_E_VALUE, "multiple of kblock"),
    ({}, dict(segments=[(0, 100, 0), (64, 64, 1)]), sa.SA_E_VALUE, "inside the previous segment"),
    ({}, dict(segments=[(0, 64, 0), (192, 100, 1)]), sa.SA_E_VALUE, "rows 100 outside"),
    ({}, dict(segments=[(0, 64, 0)], prefix_tokens=64), sa.SA_E_VALUE, "prefix_tokens must be 0"),
    ({}, dict(segments=[(64 * x, 1, 0) for x in range(17)]), sa.SA_E_VALUE, "n_segments"),
    (dict(Lkv=6146 * 64, lkv_valid=6146 * 64, Lv=6146 * 64), {}, sa.SA_E_SHAPE, "at most 6144 key blocks"),
    (dict(Lkv=6146 * 64, lkv_valid=6146 * 64, Lv=6146 * 64), dict(rule=sa.SA_RULE_TOPK, sparsity=0.5),
     sa.SA_E_SHAPE, "at most 6144 key blocks"),
])
def test_route_validation(dims_kw, prm_kw, code, msg):
    assert _route(_dims(**dims_kw), _prm(**prm_kw)) == code
    assert msg in _err()


def test_route_needs_workspace_for_sol_rule():
    dims, prm = _dims(), _prm()
    need = _lib().sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 0)
    assert need == 2 * 2 * 128 + 4 * 2 * 128   # query and key column sums, two int8 digit planes each
    assert _route(dims, prm) == sa.SA_E_WORKSPACE
    assert _route(dims, prm, ws=ctypes.c_void_p(256), wsb=need - 1) == sa.SA_E_WORKSPACE
    assert _route(dims, prm, ws=ctypes.c_void_p(260), wsb=need) == sa.SA_E_ALIGN
    assert _lib().sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 1) == 0


def test_route_explicit_map_granularity():
    assert _route(_dims(), _prm(map_kblock=96), em=ctypes.c_void_p(256)) == sa.SA_E_VALUE
    assert _route(_dims(), _prm(centroids_per_block=2), em=ctypes.c_void_p(256), G_out=False) == sa.SA_E_NULL


def test_valid_call_without_gpu_reports_device_error():
    """Arguments that pass validation reach the device check, which fails
    cleanly in a container without a GPU (and would reject a non-gfx950 GPU).
    The pointers are dummies, so this only runs where no GPU is visible."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("dummy pointers: meaningful only without a GPU")
    dims, prm = _dims(), _prm()
    need = _lib().sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 0)
    rc = _route(dims, prm, ws=ctypes.c_void_p(256), wsb=need)
    assert rc == sa.SA_E_DEVICE
    assert "device" in _err()
    assert _lib().sa_device_check(0) == sa.SA_E_DEVICE


def test_fwd_validation():
    lib = _lib()
    p = ctypes.c_void_p(256)
    dims, prm = _dims(), _prm()
    args = lambda **kw: dict(dict(v_dtype=sa.SA_BF16, sm=0.088, odt=sa.SA_F32), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.sparse_attn_fwd(p, p, p, p, p, a["v_dtype"], None, None, ctypes.byref(dims), ctypes.byref(prm), p,
                                   p, p, p, a["sm"], p, a["odt"], None, None)
    assert call(v_dtype=7) == sa.SA_E_VALUE
    assert call(v_dtype=sa.SA_INT8) == sa.SA_E_NULL      # INT8 V needs scales
    assert call(sm=0.0) == sa.SA_E_VALUE
    assert call(sm=float("nan")) == sa.SA_E_VALUE
    assert call(odt=sa.SA_INT8) == sa.SA_E_VALUE


def test_gather_validation():
    lib = _lib()
    p = ctypes.c_void_p(256)
    src_ok = (ctypes.c_int32 * 7)(0, 1, 0, 1, 1, 0, 1)
    src_bad = (ctypes.c_int32 * 7)(0, 1, 2, 1, 1, 0, 1)
    assert lib.gather_virtual_kv(p, 1, 2, 2048, 2, 128, src_bad, 7, p, p, 0, 44, 64, p, p, p, None) == sa.SA_E_VALUE
    assert "src_map[2]" in _err()
    assert lib.gather_virtual_kv(p, 1, 2, 2048, 2, 128, src_ok, 17, p, p, 0, 44, 64, p, p, p, None) == sa.SA_E_SHAPE
    assert lib.gather_virtual_kv(p, 1, 2, 2048, 2, 128, src_ok, 7, p, p, 1, 44, 64, p, p, p, None) == sa.SA_E_VALUE
    assert lib.gather_virtual_kv(p, 1, 2, 2000, 2, 128, src_ok, 7, p, p, 0, 44, 64, p, p, p, None) == sa.SA_E_SHAPE
    assert lib.gather_virtual_kv(p, 1, 2, 2048, 2, 128, src_ok, 7, p, p, 100, 44, 64, p, p, p, None) == sa.SA_E_VALUE


def test_topk_rule_without_centroids_passes_validation():
    """The fixed-sparsity rule accepts G = 0 (pruned blocks are dropped) and then
    needs no centroid outputs; without a GPU the call stops at the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("dummy pointers: meaningful only without a GPU")
    dims, prm = _dims(), _prm(rule=sa.SA_RULE_TOPK, sparsity=0.75, centroids_per_block=0)
    need = _lib().sparse_attn_route_workspace_size(ctypes.byref(dims), ctypes.byref(prm), 0)
    assert need > 0
    assert _route(dims, prm, ws=ctypes.c_void_p(256), wsb=need, G_out=False) == sa.SA_E_DEVICE


def test_cache_append_validation():
    lib = _lib()
    p = ctypes.c_void_p(256)
    ok = dict(rows=256, d=128, valid=256, R=128, slots=4, first=0)
    def call(**kw):
        a = dict(ok, **kw)
        return lib.kv_cache_append_int8(p, 0, 0, 128, 1, 1, a["rows"], a["d"], a["valid"], a["R"], p, p, a["slots"],
                                         a["first"], None)
    assert call(rows=200, valid=200) == sa.SA_E_SHAPE          # not whole slabs
    assert call(slots=1) == sa.SA_E_SHAPE                      # 2 slabs into a ring of 1
    assert call(first=4) == sa.SA_E_VALUE
    assert call(first=-1) == sa.SA_E_VALUE
    assert call(R=32) == sa.SA_E_VALUE
    assert call(valid=300) == sa.SA_E_SHAPE
    assert call(d=96) == sa.SA_E_SHAPE
    assert lib.kv_cache_append_int8(None, 0, 0, 128, 1, 1, 256, 128, 256, 128, p, p, 4, 0, None) == sa.SA_E_NULL


def test_fwd_float_validation():
    lib = _lib()
    p = ctypes.c_void_p(256)
    dims, prm = _dims(), _prm()
    call = lambda **kw: lib.sparse_attn_fwd_float(kw.get("q", p), p, p, None, ctypes.byref(kw.get("dims", dims)),
                                                  ctypes.byref(kw.get("prm", prm)), p, p, p, p, kw.get("sm", 0.088), p,
                                                  kw.get("odt", sa.SA_F32), None, None)
    assert call(q=None) == sa.SA_E_NULL
    assert call(q=ctypes.c_void_p(8)) == sa.SA_E_ALIGN
    assert call(sm=0.0) == sa.SA_E_VALUE
    assert call(odt=sa.SA_INT8) == sa.SA_E_VALUE
    assert call(dims=_dims(d=96)) == sa.SA_E_SHAPE
    assert call(prm=_prm(segments=[(0, 64, 0), (100, 10, 1)])) == sa.SA_E_VALUE


def test_forward_rejects_heads_over_4gib():
    """With a V block table, V may be longer than the key sequence; a head's
    bf16 V of 2^24 rows x 256 B would overflow the kernels' 32-bit buffer
    offsets, and both forwards refuse it before touching memory."""
    lib = _lib()
    p = ctypes.c_void_p(256)
    big = _dims(Lq=256, Lkv=256, lkv_valid=256, Lv=1 << 24, d=128)
    prm = _prm(centroids_per_block=0)
    rc = lib.sparse_attn_fwd(p, p, p, p, p, sa.SA_BF16, None, p, ctypes.byref(big), ctypes.byref(prm), p, None,
                             None, None, 0.088, p, sa.SA_F32, None, None)
    assert rc == sa.SA_E_SHAPE and "4 GiB" in _err()
    rc = lib.sparse_attn_fwd_float(p, p, p, p, ctypes.byref(big), ctypes.byref(prm), p, None, None, None, 0.088, p,
                                   sa.SA_F32, None, None)
    assert rc == sa.SA_E_SHAPE and "4 GiB" in _err()
