"""GPU parity of the 4-bit indexer variant ("FP4 Main KV Cache To Halve Storage Again": the
indexer queries and keys are 4-bit): E2M1 keys with one absmax/6 scale per row, the query
quantised to E2M1 per (token, head), the contraction on the FP4 form of the 32x32x64 MFMA.

Bars as for the fp8 indexer: key codes and scales bit-exact; scores within 1e-5 of the
per-element sum of |terms| (fp32 accumulation of exact 4-bit products); Top-K by the
near-tie rule; layer groups by the near-tie rule and the attention bar.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (DEV, build_cache, check_topk_near_tie, fp4_score_bound, max_abs_rel, one_hot_keys,
                     single_head_edge_queries, to_dev)

pytestmark = pytest.mark.gpu

csa2 = pytest.importorskip("compressed_sparse_attention_csa2_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert csa2.device_check() == 0, "not a gfx950 device"


def fp4_keys(k, n_max=None):
    B, n, dk = k.shape
    n_max = n if n_max is None else n_max
    cr, sr = oracle.quantize_fp4_rows(k, n_max=n_max)
    codes = torch.zeros((B, n_max, dk // 2), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((B, n_max), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_PER_TOKEN, to_dev(k), codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), sr) and np.array_equal(codes.cpu().numpy(), cr)
    return codes, scales, cr, sr


def test_quantize_fp4_rows_bitexact_special_values_bf16_append():
    wl = workloads.workload("full64k")
    k = np.stack([wl.index_keys(b, rows=2500) for b in range(2)])
    k[0, 0, :8] = [6.0, 0.0, -0.0, 1e-6, -1e-6, 0.25, 0.75, 100.0]
    k[0, 1, :] = 0.0
    codes, scales, cr, sr = fp4_keys(k, n_max=2600)
    new = torch.from_numpy(np.random.default_rng(3).normal(size=(2, 7, 64)).astype(np.float32)).to(torch.bfloat16)
    n0 = np.array([2500, 2593], np.int32)
    oracle.quantize_fp4_rows(new.float().numpy(), n_max=2600, n0=n0, codes=cr, scales=sr)
    csa2.quantize_kv(csa2.FMT_FP4_PER_TOKEN, new.to(DEV), codes, scales, n0=to_dev(n0))
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), sr) and np.array_equal(codes.cpu().numpy(), cr)


@pytest.mark.parametrize("T,causal", [(1, False), (3, False), (9, True)])
def test_index_score_fp4(T, causal):
    wl = workloads.workload("full64k", B=2, T=T)
    n = 5000
    k = np.stack([wl.index_keys(b, rows=n) for b in range(2)])
    codes, scales, cr, sr = fp4_keys(k)
    q, w = wl.index_query(), wl.head_weights()
    nk = np.array([n, 3777], np.int32)
    ql = (np.array([[4000], [2000]]) + np.arange(T)[None]).astype(np.int32) if causal else None
    ref = oracle.index_score(oracle.PREC_FP4, q, w, cr, sr, nk, q_limit=ql)
    got = csa2.index_score(csa2.PREC_FP4, to_dev(q, torch.bfloat16), to_dev(w), codes, scales, to_dev(nk),
                           q_limit=None if ql is None else to_dev(ql)).cpu().numpy()
    vis = np.isfinite(ref)
    assert np.array_equal(vis, np.isfinite(got))
    bound = fp4_score_bound(q, w, cr, sr)
    assert np.all(np.abs(got[vis] - ref[vis]) <= 1e-5 * bound[vis] + 1e-30)
    idx = csa2.index_topk(csa2.PREC_FP4, to_dev(q, torch.bfloat16), to_dev(w), codes, scales, to_dev(nk), 512,
                          q_limit=None if ql is None else to_dev(ql))
    check_topk_near_tie(idx.cpu().numpy(), ref, 512)


@pytest.mark.parametrize("with_cand", [False, True])
def test_index_query_codes_exact_fp4(with_cand):
    """The E2M1 query quantisation inside the 4-bit scoring kernel, code for code: one-hot
    keys and one-head queries make every score a single product of one query code's value
    and the scales (a differing code moves it by at least 1/4 of itself); bar 1e-6 relative.
    Heads cover scales below 2^-92, six decades inside a head, 1e30 and all-zero heads."""
    B = 32
    wl = workloads.workload("full64k", B=B)
    n = 128
    codes, scales, cr, sr = fp4_keys(one_hot_keys(B, n))
    q, w = single_head_edge_queries(wl.index_query()), wl.head_weights()
    nk = np.full(B, n, np.int32)
    cand = None
    if with_cand:
        rng = np.random.default_rng(6)
        cand = np.stack([rng.permutation(np.concatenate([np.arange(n), np.full(30, -1)])) for _ in range(B)])
        cand = cand[:, None].astype(np.int32)
    ref = oracle.index_score(oracle.PREC_FP4, q, w, cr, sr, nk, cand=cand)
    got = csa2.index_score(csa2.PREC_FP4, to_dev(q, torch.bfloat16), to_dev(w), codes, scales, to_dev(nk),
                           cand=None if cand is None else to_dev(cand)).cpu().numpy()
    vis = np.isfinite(ref)
    assert np.array_equal(vis, np.isfinite(got))
    assert np.all(np.abs(got[vis] - ref[vis]) <= 1e-6 * np.abs(ref[vis]))
    assert np.count_nonzero(ref[vis]) > vis.sum() // 3


def test_index_score_fp4_candidates_and_fp32_query():
    wl = workloads.workload("full64k", B=2)
    n = 3000
    k = np.stack([wl.index_keys(b, rows=n) for b in range(2)])
    codes, scales, cr, sr = fp4_keys(k)
    q, w = wl.index_query(), wl.head_weights()
    rng = np.random.default_rng(8)
    cand = rng.integers(-1, n, size=(2, 1, 777)).astype(np.int32)
    nk = np.array([n, 2500], np.int32)
    ref = oracle.index_score(oracle.PREC_FP4, q, w, cr, sr, nk, cand=cand)
    got = csa2.index_score(csa2.PREC_FP4, to_dev(q), to_dev(w), codes, scales, to_dev(nk),
                           cand=to_dev(cand)).cpu().numpy()
    vis = np.isfinite(ref)
    assert np.array_equal(vis, np.isfinite(got))
    assert np.allclose(got[vis], ref[vis], rtol=1e-4, atol=1e-4 * np.abs(ref[vis]).max())


@pytest.mark.parametrize("pool", [None, (8, 128)])
def test_layer_group_fp4_indexer(pool):
    wl = workloads.workload("group128k", B=3, N=20000, K=256)
    c = build_cache(wl)
    kf = np.stack([wl.index_keys(b, rows=wl.N) for b in range(3)])
    codes, scales, cr, sr = fp4_keys(kf)
    nk = np.array([20000, 15001, 900], np.int32)
    modes = ["full", "reindex", "reuse"]
    layers, ref_layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        ref_layers.append(dict(mode=m, q_idx=qi, w=w, q_attn=qa))
        L = dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16))
        if m == "full" and pool:
            L["pool"] = torch.full((3, pool[0] * pool[1]), -7, dtype=torch.int32, device=DEV)
        layers.append(L)
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], codes, scales, wl.K, wl.softmax_scale,
                            prec=csa2.PREC_FP4, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g_idx, gpool = None, None
    for i, (L, RL) in enumerate(zip(layers, ref_layers)):
        if L["mode"] != "reuse":
            g_idx = L["idx"].cpu().numpy()
            if L["mode"] == "full" or pool is None:
                s = oracle.index_score(oracle.PREC_FP4, RL["q_idx"], RL["w"], cr, sr, nk)
                check_topk_near_tie(g_idx, s, wl.K)
                if pool:
                    gpool = L["pool"].cpu().numpy()
            else:
                fs = oracle.index_score(oracle.PREC_FP4, RL["q_idx"], RL["w"], cr, sr, nk, cand=gpool[:, None])
                full = np.full((3, 1, wl.N), -np.inf)
                for b in range(3):
                    ok = gpool[b] >= 0
                    full[b, 0, gpool[b][ok]] = fs[b, 0][ok]
                check_topk_near_tie(g_idx, full, wl.K)
        ro, _ = oracle.sparse_attend(RL["q_attn"], c["codes_ref"], c["scales_ref"], g_idx, wl.softmax_scale)
        assert max_abs_rel(L["out"].cpu().numpy(), ro) <= 2e-3, i
