"""Pins for the oracle's forward pass (CPU only).

Configure Sol Sparse Attention, "How it works": kept blocks are computed exactly
on the INT8 Q/K; a skipped block stands in as a single 64-token centroid (1x64) or
two 32-token centroids (2x32) that still contribute to the softmax.  Configure H3
Static Virtual KV, mode list ("residual"): centroids share the online softmax
with the exact blocks.  FlashVSR Sparge Attention, opening section: a dense
masked kernel is slower but correct, and is the intended fallback.
"""
import math

import numpy as np
import torch

import workloads as W
from workloads import bf16_bits, bf16_to_f32, EXACT, CENTROID, DROP


def _deq(codes, scales, rows):
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), rows, axis=-1)[..., None]


def _sdpa(q, k, v, mask):
    """float64 torch SDPA (a library routine, not our formula); mask True = attend."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=t(mask))
    return o.numpy()


def _blocks_to_rows(out, nQB):
    B_H = out.shape[0] // nQB
    return out.reshape(B_H, nQB * 128, -1)


def test_all_exact_is_softmax_attention(orc):
    wl = W.tiny_sol(seed=21, H=2, L=512, d=64, valid=450)
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, 64)
    r = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=float("inf"), G=1)
    out, lse, _ = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                              vbar=r["vbar"], count=r["count"], v_bits=wl.v)
    qd, kd = _deq(q8, qs, 128)[0], _deq(k8, ks, 64)[0]
    vd = bf16_to_f32(wl.v)[0].astype(np.float64)
    mask = np.zeros((512, 512), bool)
    mask[:, :wl.lkv_valid] = True
    ref = _sdpa(qd, kd, vd, mask)
    got = _blocks_to_rows(out, 4)
    assert np.abs(got[:, :wl.lq_valid] - ref[:, :wl.lq_valid]).max() < 1e-12
    assert not got[:, wl.lq_valid:].any()
    assert np.isneginf(lse.reshape(2, 512)[:, wl.lq_valid:]).all()
    # lse against the definition with a library logsumexp
    logits = np.einsum("hqd,hkd->hqk", qd, kd) / math.sqrt(64)
    ref_lse = torch.logsumexp(torch.from_numpy(logits[:, :, :wl.lkv_valid]), dim=-1).numpy()
    assert np.abs(lse.reshape(2, 512)[:, :wl.lq_valid] - ref_lse[:, :wl.lq_valid]).max() < 1e-10


def test_lcsa_equals_masked_dense(orc):
    wl = W.config(2, small=True)
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, 128)
    v8, vs = orc.quantize(wl.v, wl.lkv_valid, 128)
    r = orc.route(q8, k8, ks, 128, wl.lq_valid, wl.lkv_valid, v8=v8, v_scale=vs, G=0, kblock=128,
                  explicit_map=wl.explicit_map, map_kblock=128)
    out, _, _ = orc.forward(q8, qs, k8, ks, 128, wl.lq_valid, wl.lkv_valid, r["map"], v8=v8, v_scale=vs,
                            kblock=128, G=0)
    nQB = wl.Lq // 128
    got = _blocks_to_rows(out, nQB)
    qd, kd, vd = _deq(q8, qs, 128)[0], _deq(k8, ks, 128)[0], _deq(v8, vs, 128)[0]
    for h in range(wl.H):
        tok = np.kron(wl.explicit_map[0, h] == EXACT, np.ones((128, 128), bool))
        ref = _sdpa(qd[h:h + 1], kd[h:h + 1], vd[h:h + 1], tok)[0]
        assert np.abs(got[h] - ref).max() < 1e-12


def _one_block_case(n_valid=64, identical=None, seed=0, d=64, Lq=128):
    """Lq queries, one key block of 64 rows (n_valid of them valid)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, Lq, d), dtype=np.float32)
    k = rng.standard_normal((1, 1, 64, d), dtype=np.float32)
    v = rng.standard_normal((1, 1, 64, d), dtype=np.float32)
    if identical == "block":
        k[0, 0, :] = k[0, 0, 0]
    elif identical == "halves":
        k[0, 0, :32] = k[0, 0, 0]
        k[0, 0, 32:] = k[0, 0, 40]
    return bf16_bits(q), bf16_bits(k), bf16_bits(v), n_valid


def _run_forced(orc, q, k, v, n_valid, state, G, Lq=128):
    q8, qs = orc.quantize(q, Lq, 128)
    k8, ks = orc.quantize(k, n_valid, 64)
    nQB = Lq // 128
    em = np.full((1, 1, nQB, 1), state, np.uint8)
    r = orc.route(q8, k8, ks, 64, Lq, n_valid, v_bits=v, G=G, kblock=64, explicit_map=em, map_kblock=64)
    out, lse, _ = orc.forward(q8, qs, k8, ks, 64, Lq, n_valid, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                              count=r["count"], v_bits=v, G=G)
    return out.reshape(Lq, -1), r


def test_single_centroid_block_outputs_vbar(orc):
    q, k, v, n = _one_block_case()
    out, r = _run_forced(orc, q, k, v, n, CENTROID, 1)
    vbar = bf16_to_f32(v)[0, 0].astype(np.float64).mean(0)
    assert np.abs(out - vbar[None]).max() < 1e-14


def test_identical_keys_centroid_equals_exact(orc):
    q, k, v, n = _one_block_case(identical="block", seed=1)
    ex, _ = _run_forced(orc, q, k, v, n, EXACT, 1)
    ce, _ = _run_forced(orc, q, k, v, n, CENTROID, 1)
    assert np.abs(ex - ce).max() < 1e-12


def test_2x32_identical_halves(orc):
    q, k, v, n = _one_block_case(identical="halves", seed=2)
    ex, _ = _run_forced(orc, q, k, v, n, EXACT, 1)
    c2, _ = _run_forced(orc, q, k, v, n, CENTROID, 2)
    c1, _ = _run_forced(orc, q, k, v, n, CENTROID, 1)
    assert np.abs(ex - c2).max() < 1e-12
    assert np.abs(ex - c1).max() > 1e-3       # one centroid cannot represent two distinct keys


def test_partial_block_needs_count_weight(orc):
    # 40 valid identical keys in a 64-row block plus an exact block elsewhere:
    # the centroid must carry weight 40 to reproduce the exact result.
    rng = np.random.default_rng(3)
    d = 64
    q = bf16_bits(rng.standard_normal((1, 1, 128, d), dtype=np.float32))
    k = rng.standard_normal((1, 1, 128, d), dtype=np.float32)
    k[0, 0, 64:] = k[0, 0, 64]
    k = bf16_bits(k)
    v = bf16_bits(rng.standard_normal((1, 1, 128, d), dtype=np.float32))
    n_valid = 104
    q8, qs = orc.quantize(q, 128, 128)
    k8, ks = orc.quantize(k, n_valid, 64)
    outs = {}
    for st in (EXACT, CENTROID):
        em = np.array([[[[EXACT, st]]]], np.uint8)
        r = orc.route(q8, k8, ks, 64, 128, n_valid, v_bits=v, G=1, kblock=64, explicit_map=em, map_kblock=64)
        assert r["count"][0, 0, 1, 0] == 40
        outs[st], _, _ = orc.forward(q8, qs, k8, ks, 64, 128, n_valid, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                                     count=r["count"], v_bits=v)
    assert np.abs(outs[EXACT] - outs[CENTROID]).max() < 1e-12
    # the same centroid with weight 1 would give a visibly different answer
    r["count"][0, 0, 1, 0] = 1.0
    w1, _, _ = orc.forward(q8, qs, k8, ks, 64, 128, n_valid, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                           count=r["count"], v_bits=v)
    assert np.abs(w1 - outs[EXACT]).max() > 1e-2


def test_outputs_in_hull_and_drop_rows(orc):
    wl = W.config(3, small=True)
    res = orc.run(wl)
    vmin = bf16_to_f32(wl.v).min()
    vmax = bf16_to_f32(wl.v).max()
    assert res["out"].min() >= vmin - 1e-12 and res["out"].max() <= vmax + 1e-12
    # an all-drop row gives zeros and lse = -inf
    m = res["map"].copy()
    m[0, 0, 0, :] = DROP
    out, lse, _ = orc.forward(res["q8"], res["q_scale"], res["k8"], res["k_scale"], 64, wl.lq_valid,
                              wl.lkv_valid, m, kbar=res["kbar"], vbar=res["vbar"], count=res["count"],
                              v_bits=wl.v, sel=[0])
    assert not out.any() and np.isneginf(lse).all()


def test_centroid_mix_matches_explicit_logit_softmax(orc):
    """A small routed case against a float64 softmax over an explicitly listed
    set of columns (exact keys plus centroid columns with log-count bias),
    evaluated with torch.softmax."""
    wl = W.tiny_sol(seed=31, H=1, L=256, d=64)
    q8, qs = orc.quantize(wl.q, 256, 128)
    k8, ks = orc.quantize(wl.k, 256, 64)
    r = orc.route(q8, k8, ks, 64, 256, 256, v_bits=wl.v, tau=0.0, G=2)
    assert (r["map"] == CENTROID).any() and (r["map"] == EXACT).any()
    out, _, _ = orc.forward(q8, qs, k8, ks, 64, 256, 256, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                            count=r["count"], v_bits=wl.v, G=2)
    qd, kd = _deq(q8, qs, 128)[0, 0], _deq(k8, ks, 64)[0, 0]
    vd = bf16_to_f32(wl.v)[0, 0].astype(np.float64)
    for i in range(2):
        cols_k, cols_v, bias = [], [], []
        for j in range(4):
            if r["map"][0, 0, i, j] == EXACT:
                cols_k += list(kd[j * 64:(j + 1) * 64]); cols_v += list(vd[j * 64:(j + 1) * 64]); bias += [0.0] * 64
            elif r["map"][0, 0, i, j] == CENTROID:
                for g in range(2):
                    cols_k.append(kd[j * 64 + g * 32:j * 64 + g * 32 + 32].mean(0))
                    cols_v.append(vd[j * 64 + g * 32:j * 64 + g * 32 + 32].mean(0))
                    bias.append(math.log(32))
        logit = qd[i * 128:(i + 1) * 128] @ np.array(cols_k).T / 8.0 + np.array(bias)
        p = torch.softmax(torch.from_numpy(logit), dim=-1).numpy()
        ref = p @ np.array(cols_v)
        assert np.abs(out[i] - ref).max() < 1e-12


# ---------------------------------------------------------------------------
# Floating QK path (Configure Sol Sparse Attention, "How it works": with a
# floating dense backend the exact blocks run in floating point, not W8A8).
# ---------------------------------------------------------------------------

def test_float_path_all_exact_is_softmax_attention_on_bf16(orc):
    wl = W.tiny_sol(seed=23, H=2, L=512, d=64, valid=450)
    q8, qs = orc.quantize(wl.q, wl.lq_valid, 128)
    k8, ks = orc.quantize(wl.k, wl.lkv_valid, 64)
    r = orc.route(q8, k8, ks, 64, wl.lq_valid, wl.lkv_valid, v_bits=wl.v, tau=float("inf"), G=1)
    out, lse, _ = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                              vbar=r["vbar"], count=r["count"], v_bits=wl.v, q_bits=wl.q, k_bits=wl.k)
    qf, kf, vf = (bf16_to_f32(t)[0].astype(np.float64) for t in (wl.q, wl.k, wl.v))
    mask = np.zeros((512, 512), bool)
    mask[:, :wl.lkv_valid] = True
    ref = _sdpa(qf, kf, vf, mask)
    got = _blocks_to_rows(out, 4)
    assert np.abs(got[:, :wl.lq_valid] - ref[:, :wl.lq_valid]).max() < 1e-12
    logits = np.einsum("hqd,hkd->hqk", qf, kf) / math.sqrt(64)
    ref_lse = torch.logsumexp(torch.from_numpy(logits[:, :, :wl.lkv_valid]), dim=-1).numpy()
    assert np.abs(lse.reshape(2, 512)[:, :wl.lq_valid] - ref_lse[:, :wl.lq_valid]).max() < 1e-10
    # the INT8 path differs from it by the quantization error only
    o8, _, _ = orc.forward(q8, qs, k8, ks, 64, wl.lq_valid, wl.lkv_valid, r["map"], kbar=r["kbar"],
                           vbar=r["vbar"], count=r["count"], v_bits=wl.v)
    diff = np.abs(_blocks_to_rows(o8, 4) - got)[:, :wl.lq_valid]
    assert 0 < diff.max() < 0.1


def test_float_path_single_centroid_block_outputs_vbar(orc):
    q, k, v, n = _one_block_case()
    Lq = q.shape[2]
    q8, qs = orc.quantize(q, Lq, 128)
    k8, ks = orc.quantize(k, n, 64)
    em = np.full((1, 1, Lq // 128, 1), CENTROID, np.uint8)
    r = orc.route(q8, k8, ks, 64, Lq, n, v_bits=v, G=1, kblock=64, explicit_map=em, map_kblock=64)
    out, _, _ = orc.forward(q8, qs, k8, ks, 64, Lq, n, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                            count=r["count"], v_bits=v, G=1, q_bits=q, k_bits=k)
    vbar = bf16_to_f32(v)[0, 0, :n].astype(np.float64).mean(0)
    assert np.abs(out.reshape(Lq, -1) - vbar[None]).max() < 1e-14


def test_float_path_centroid_mix_matches_explicit_logit_softmax(orc):
    """Floating QK path with exact keys and several 2x32 centroid columns per
    row, against a float64 torch.softmax over explicitly listed columns: exact
    keys with logit q.k / sqrt(d) on the bf16 values, centroid columns with
    logit q.kbar / sqrt(d) + ln(count) on the bf16 query, kbar the mean of the
    dequantized INT8 keys of the group (the centroids are routed on the codes
    whatever the backend).  Several centroid columns with different logits per
    row make the logit's scale and its query operand matter."""
    wl = W.tiny_sol(seed=37, H=1, L=512, d=64, valid=500)
    q8, qs = orc.quantize(wl.q, 500, 128)
    k8, ks = orc.quantize(wl.k, 500, 64)
    r = orc.route(q8, k8, ks, 64, 500, 500, v_bits=wl.v, tau=-0.3, G=2)
    cen = (r["map"] == CENTROID).sum(-1)
    assert cen.min() >= 2 and (r["map"] == EXACT).sum(-1).min() >= 2
    out, lse, _ = orc.forward(q8, qs, k8, ks, 64, 500, 500, r["map"], kbar=r["kbar"], vbar=r["vbar"],
                              count=r["count"], v_bits=wl.v, G=2, q_bits=wl.q, k_bits=wl.k)
    qf, kf, vf = (bf16_to_f32(t)[0, 0].astype(np.float64) for t in (wl.q, wl.k, wl.v))
    kd = _deq(k8, ks, 64)[0, 0]
    for i in range(4):
        cols_k, cols_v, bias = [], [], []
        for j in range(8):
            rows = [u for u in range(j * 64, j * 64 + 64) if u < 500]
            if r["map"][0, 0, i, j] == EXACT:
                cols_k += [kf[u] for u in rows]; cols_v += [vf[u] for u in rows]; bias += [0.0] * len(rows)
            elif r["map"][0, 0, i, j] == CENTROID:
                for g in range(2):
                    grp = [u for u in rows if j * 64 + g * 32 <= u < j * 64 + g * 32 + 32]
                    if not grp:
                        continue
                    cols_k.append(kd[grp].mean(0)); cols_v.append(vf[grp].mean(0)); bias.append(math.log(len(grp)))
        r1 = min(128, 500 - i * 128)
        logit = qf[i * 128:i * 128 + r1] @ np.array(cols_k).T / 8.0 + np.array(bias)
        p = torch.softmax(torch.from_numpy(logit), dim=-1).numpy()
        ref = p @ np.array(cols_v)
        assert np.abs(out[i, :r1] - ref).max() < 1e-12
        ref_lse = torch.logsumexp(torch.from_numpy(logit), dim=-1).numpy()
        assert np.abs(lse[i, :r1] - ref_lse).max() < 1e-10
