"""Pins of the oracle's sparse attention, layer modes and two-level indexer.

Attention over the selected entries is softmax attention with the dequantised entry as
both key and value.  With every entry selected it must equal dense attention (torch,
float64); K = 1 and q = 0 have closed forms; the order of the index list does not matter;
splitting the selected set and merging by log-sum-exp gives the same result.
Modes follow "The Three Modes Full Reindex And Reuse" (paper notes) and the 3.3 mode table
of the Chinese reading; the two-level indexer follows the configuration's block-mean
reading and must reduce to the flat Top-K when every block is kept.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def _dequant_all(codes, s):
    # independent FP4 decode: low nibble = even channel; a dequantised value is the fp32
    # product E2M1(code) * s (exact in fp64, then rounded once to fp32)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], codes.shape[1], -1)
    return (E2M1[nib] * s[:, None, :].astype(np.float64)).astype(np.float32).astype(np.float64)


def _cache(wl, n):
    x = np.stack([wl.main_kv(b, rows=n) for b in range(wl.B)])
    return oracle.quantize_fp4(x)


def test_full_selection_equals_dense_attention():
    wl = workloads.workload("tiny", N=96)
    codes, s = _cache(wl, 96)
    q = wl.attn_query()
    idx = np.arange(96, dtype=np.int32)[None, None]
    out, lse = oracle.sparse_attend(q, codes, s, idx, wl.softmax_scale)
    V = torch.from_numpy(_dequant_all(codes, s))[0]                       # [N][D]
    Q = torch.from_numpy(q).double()[0, 0]                                 # [Hq][D]
    logits = wl.softmax_scale * Q @ V.T
    ref = torch.softmax(logits, dim=-1) @ V
    assert np.allclose(out[0, 0], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[0, 0], torch.logsumexp(logits, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_k1_returns_the_row_and_q0_returns_the_mean():
    wl = workloads.workload("tiny", N=64)
    codes, s = _cache(wl, 64)
    V = _dequant_all(codes, s)[0]
    q = wl.attn_query()
    out, _ = oracle.sparse_attend(q, codes, s, np.array([[[17]]], np.int32), wl.softmax_scale)
    assert np.array_equal(out[0, 0], np.broadcast_to(V[17], out[0, 0].shape))
    sel = np.array([[[3, 9, 40, 41, -1]]], np.int32)
    out0, lse0 = oracle.sparse_attend(np.zeros_like(q), codes, s, sel, wl.softmax_scale)
    assert np.allclose(out0[0, 0], V[[3, 9, 40, 41]].mean(axis=0), rtol=1e-13, atol=1e-13)
    assert np.allclose(lse0, np.log(4.0))


def test_permutation_invariance_and_empty_set():
    wl = workloads.workload("tiny", N=128)
    codes, s = _cache(wl, 128)
    q = wl.attn_query()
    rng = np.random.default_rng(3)
    sel = rng.choice(128, 40, replace=False).astype(np.int32)[None, None]
    a, la = oracle.sparse_attend(q, codes, s, sel, wl.softmax_scale)
    b, lb = oracle.sparse_attend(q, codes, s, sel[..., ::-1].copy(), wl.softmax_scale)
    assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12
    e, le = oracle.sparse_attend(q, codes, s, np.full((1, 1, 8), -1, np.int32), wl.softmax_scale)
    assert np.all(e == 0) and np.all(np.isneginf(le))


@pytest.mark.parametrize("parts", [2, 3, 7])
def test_split_and_lse_merge_equals_whole(parts):
    wl = workloads.workload("tiny", N=200)
    codes, s = _cache(wl, 200)
    q = wl.attn_query()
    sel = np.random.default_rng(parts).choice(200, 64, replace=False).astype(np.int32)
    whole, lw = oracle.sparse_attend(q, codes, s, sel[None, None], wl.softmax_scale)
    outs, lses = [], []
    for chunk in np.array_split(sel, parts):
        pad = np.full(64, -1, np.int32)
        pad[:len(chunk)] = chunk
        o, l = oracle.sparse_attend(q, codes, s, pad[None, None], wl.softmax_scale)
        outs.append(o)
        lses.append(l)
    L = np.logaddexp.reduce(np.stack(lses), axis=0)
    merged = sum(np.exp(l - L)[..., None] * o for o, l in zip(outs, lses))
    assert np.max(np.abs(merged - whole)) < 1e-12 and np.max(np.abs(L - lw)) < 1e-12


def _group_inputs(wl, n):
    k = np.stack([wl.index_keys(b, rows=n) for b in range(wl.B)])
    k8, ks = oracle.quantize_fp8(k)
    codes, s = _cache(wl, n)
    cache = dict(k=k8, k_scale=ks, n_keys=np.full(wl.B, n, np.int32), codes=codes, scales=s)
    return cache


def test_modes_reuse_reindex_invariants():
    wl = workloads.workload("group128k", N=1024, B=2, K=64)
    cache = _group_inputs(wl, 1024)
    layers = [dict(mode=m, q_idx=wl.index_query(i), w=wl.head_weights(i), q_attn=wl.attn_query(i))
              for i, m in enumerate(["full", "reindex", "reuse", "reuse"])]
    res = oracle.layer_group(layers, cache, oracle.PREC_FP8, wl.K, wl.softmax_scale)
    # Reuse takes the most recent indexing layer's indices unchanged
    assert res[2]["idx"] is res[1]["idx"] and res[3]["idx"] is res[1]["idx"]
    assert not np.array_equal(res[0]["idx"], res[1]["idx"])
    # Reindex fed Full's query and weights reproduces Full's indices
    same = [dict(layers[0]), dict(layers[0], mode="reindex")]
    r2 = oracle.layer_group(same, cache, oracle.PREC_FP8, wl.K, wl.softmax_scale)
    assert np.array_equal(r2[0]["idx"], r2[1]["idx"])
    # group output == single-layer calls composed
    s0 = oracle.index_score(oracle.PREC_FP8, layers[1]["q_idx"], layers[1]["w"], cache["k"], cache["k_scale"],
                            cache["n_keys"])
    i1 = oracle.topk(s0, wl.K)
    o3, _ = oracle.sparse_attend(layers[3]["q_attn"], cache["codes"], cache["scales"], i1, wl.softmax_scale)
    assert np.array_equal(res[1]["idx"], i1) and np.array_equal(res[3]["out"], o3)


@pytest.mark.parametrize("modes,ok", [
    (["full"], True), (["full", "reindex", "reuse"], True), (["full", "reuse", "reindex", "reuse"], True),
    (["reuse"], False), (["reindex"], False), (["reindex", "full"], False), ([], False), (["full", "bogus"], False),
])
def test_schedule_rules(modes, ok):
    assert oracle.check_schedule(modes) == ok


def test_pages_38_layer_schedule_is_valid():
    # Encoder: three groups of [Full, Reuse x5]; decoder: [Full, Reuse x3] then four groups of
    # [Reindex, Reuse x3] (paper notes "Model Setup Numbers Without Jargon"; 3.3 of the reading).
    enc = (["full"] + ["reuse"] * 5) * 3
    dec = ["full"] + ["reuse"] * 3 + (["reindex"] + ["reuse"] * 3) * 4
    assert len(enc) == 18 and len(dec) == 20
    assert oracle.check_schedule(enc) and oracle.check_schedule(dec)
    assert (enc + dec).count("full") == 4 and dec.count("reindex") == 4 and (enc + dec).count("reuse") == 30


def test_hierarchical_keeping_every_block_equals_flat():
    wl = workloads.workload("hier1m", N=64 * 40, K=100)
    k8, ks = oracle.quantize_fp8(wl.index_keys(0)[None])
    nk = np.array([64 * 40 - 13], np.int32)
    kb8, kbs = oracle.coarse_keys(k8, ks, nk, 64)
    q, w = wl.index_query(), wl.head_weights()
    idx, blk = oracle.hier_select(q, w, k8, ks, kb8, kbs, nk, 64, 40, wl.K)
    flat = oracle.topk(oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, nk), wl.K)
    assert np.array_equal(idx, flat)
    assert sorted(blk[0, 0].tolist()) == list(range(40))


def test_coarse_key_of_identical_rows_is_the_row():
    wl = workloads.workload("hier1m", N=128)
    row = wl.index_keys(0, rows=1)
    k = np.repeat(row[None], 128, axis=1)                  # two blocks of identical keys
    k8, ks = oracle.quantize_fp8(k)
    kb8, kbs = oracle.coarse_keys(k8, ks, np.array([128], np.int32), 64)
    f8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    key = f8(k8[0, 0]) * ks[0, 0]
    for blk in range(2):
        coarse = f8(kb8[0, blk]) * kbs[0, blk]
        assert np.allclose(coarse, key, rtol=2 ** -4, atol=1e-6 * np.abs(key).max())


def test_coarse_mean_definition_small():
    # A partial block of 3 rows: fp32 sequential sum of fl32(sk * k) then / 3.
    k = np.zeros((1, 3, 64), np.float32)
    k[0, :, 0] = [1.0, 2.0, 4.0]
    k[0, :, 1] = [-448.0, 448.0, 0.0]
    k8, ks = oracle.quantize_fp8(k)
    kb8, kbs = oracle.coarse_keys(k8, ks, np.array([3], np.int32), 64)
    f8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    mean = f8(kb8[0, 0]) * kbs[0, 0]
    assert abs(mean[0] - 7.0 / 3) < 7.0 / 3 * 2 ** -4 and abs(mean[1]) < 1e-6
