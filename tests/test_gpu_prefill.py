"""GPU parity of the chunked-prefill path: the new tokens' main KV (bf16) is quantised to
FP4 with the cache's per-channel scales and appended, their indexer keys are quantised to
E4M3 and appended, then every new token scores the cache causally (row t sees positions
<= N_c + t), keeps its Top-K and attends over it.

The small case is checked in full. The full-size case (262144 cached + 4096 new tokens)
runs the whole batch on the GPU and checks sampled rows against the oracle.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_csa2_amd as csa2
import oracle
import workloads
from helpers import DEV, check_topk_near_tie, fp8_score_bound, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu


def _prefill_cache(wl):
    """Cache of N_c entries (COMPUTE scales) plus the T new tokens appended (GIVEN scales),
    on both sides; the bytes must agree exactly."""
    Nc, T, D, dk = wl.N, wl.T, wl.D, wl.dk
    n_max = Nc + T
    x, kf = wl.main_kv(0)[None], wl.index_keys(0)[None]
    new, newk = wl.new_kv(), wl.new_index_keys()
    n0 = np.array([Nc], np.int32)
    codes_r, scales_r = oracle.quantize_fp4(x, n_max=n_max)
    oracle.quantize_fp4(new, n_max=n_max, n0=n0, scales=scales_r, codes=codes_r)
    k8_r, ks_r = oracle.quantize_fp8(kf, n_max=n_max)
    oracle.quantize_fp8(newk, n_max=n_max, n0=n0, codes=k8_r, scales=ks_r)
    codes = torch.zeros((1, n_max, D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((1, D), dtype=torch.float32, device=DEV)
    k8 = torch.zeros((1, n_max, dk), dtype=torch.uint8, device=DEV)
    ks = torch.zeros((1, n_max), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(x), codes, scales)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf), k8, ks)
    n0d = to_dev(n0)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(new, torch.bfloat16), codes, scales,
                     scale_policy=csa2.SCALE_GIVEN, n0=n0d)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(newk), k8, ks, n0=n0d)
    torch.cuda.synchronize()
    assert np.array_equal(scales.cpu().numpy(), scales_r)
    assert np.array_equal(codes.cpu().numpy(), codes_r)
    assert np.array_equal(k8.cpu().numpy(), k8_r)
    assert np.array_equal(ks.cpu().numpy(), ks_r)
    q_limit = (Nc + np.arange(T, dtype=np.int32))[None]
    return dict(codes=codes, scales=scales, k8=k8, ks=ks, codes_r=codes_r, scales_r=scales_r, k8_r=k8_r, ks_r=ks_r,
                n_keys=np.array([n_max], np.int32), q_limit=q_limit)


def test_prefill_small_whole():
    """8192 cached + 100 new tokens (the row tiles of 8 end in a partial tile)."""
    wl = workloads.workload("prefill", N=8192, T=100)
    c = _prefill_cache(wl)
    q, w, qa = wl.index_query(), wl.head_weights(), wl.attn_query()
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    nk, ql = to_dev(c["n_keys"]), to_dev(c["q_limit"])
    ref = oracle.index_score(oracle.PREC_FP8, q, w, c["k8_r"], c["ks_r"], c["n_keys"], q_limit=c["q_limit"])
    got = csa2.index_score(csa2.PREC_FP8, qd, wd, c["k8"], c["ks"], nk, q_limit=ql).cpu().numpy()
    vis = np.isfinite(ref)
    assert np.array_equal(vis, np.isfinite(got))
    bound = fp8_score_bound(q, w, c["k8_r"], c["ks_r"])
    assert np.all(np.abs(got[vis] - ref[vis]) <= 1e-5 * bound[vis] + 1e-30)
    idx = csa2.index_topk(csa2.PREC_FP8, qd, wd, c["k8"], c["ks"], nk, wl.K, q_limit=ql)
    g = idx.cpu().numpy()
    check_topk_near_tie(g, ref, wl.K)
    assert np.all(g <= c["q_limit"][..., None])  # causal
    out, lse = csa2.sparse_attend(to_dev(qa, torch.bfloat16), c["codes"], c["scales"], idx, wl.softmax_scale,
                                  out_dtype=torch.float32)
    ro, rl = oracle.sparse_attend(qa, c["codes_r"], c["scales_r"], g, wl.softmax_scale)
    assert max_abs_rel(out.cpu().numpy(), ro) <= 2e-3


def test_prefill_full_size_sampled_rows():
    """262144 cached + 4096 new tokens; every row runs on the GPU, every 64th row plus the
    first and the last is checked against the oracle."""
    wl = workloads.WORKLOADS["prefill"]
    c = _prefill_cache(wl)
    q, w, qa = wl.index_query(), wl.head_weights(), wl.attn_query()
    nk, ql = to_dev(c["n_keys"]), to_dev(c["q_limit"])
    idx = csa2.index_topk(csa2.PREC_FP8, to_dev(q, torch.bfloat16), to_dev(w), c["k8"], c["ks"], nk, wl.K, q_limit=ql)
    out, lse = csa2.sparse_attend(to_dev(qa, torch.bfloat16), c["codes"], c["scales"], idx, wl.softmax_scale,
                                  out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = sorted(set(range(0, wl.T, 64)) | {0, wl.T - 1})
    g = idx.cpu().numpy()[:, rows]
    ref = oracle.index_score(oracle.PREC_FP8, q[:, rows], w[:, rows], c["k8_r"], c["ks_r"], c["n_keys"],
                             q_limit=c["q_limit"][:, rows])
    check_topk_near_tie(g, ref, wl.K)
    ro, rl = oracle.sparse_attend(qa[:, rows], c["codes_r"], c["scales_r"], g, wl.softmax_scale)
    o = out.float().cpu().numpy()[:, rows]
    assert np.all(np.abs(o - ro) <= 2e-3 * np.abs(ro).max() + np.abs(ro) * 2.0 ** -8)


def test_many_row_scores_equal_single_row_scores():
    """The many-row kernel (T >= 8) and the decode kernel (T = 1) take the same arithmetic
    steps, so the scores agree bit for bit."""
    wl = workloads.workload("prefill", N=3000, T=24)
    c = _prefill_cache(wl)
    q, w = wl.index_query(), wl.head_weights()
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    nk, ql = to_dev(c["n_keys"]), to_dev(c["q_limit"])
    many = csa2.index_score(csa2.PREC_FP8, qd, wd, c["k8"], c["ks"], nk, q_limit=ql)
    for t in [0, 5, 8, 17, 23]:
        one = csa2.index_score(csa2.PREC_FP8, qd[:, t:t + 1].contiguous(), wd[:, t:t + 1].contiguous(), c["k8"],
                               c["ks"], nk, q_limit=ql[:, t:t + 1].contiguous())
        assert torch.equal(one[:, 0], many[:, t]), t


def test_prefill_with_compressed_entries_m2():
    """Encoder-style compression m = 2 ("CSA2 In Simple Terms": two tokens share one stored
    entry in the encoder): entry j covers tokens 2j and 2j + 1, so the new token at position
    p sees the entries whose tokens are all at or before p, j <= (p + 1) / 2 - 1.  4096
    cached entries (8192 tokens), 64 new tokens forming 32 new entries."""
    wl = workloads.workload("prefill", N=4096, T=64)
    Nc, T, dk = wl.N, wl.T, wl.dk
    n_new = T // 2
    n_max = Nc + n_new
    kf = wl.index_keys(0, rows=n_max)[None]                      # cached and new entries' keys
    x = wl.main_kv(0, rows=n_max)[None]
    k8r, ksr = oracle.quantize_fp8(kf)
    cr, sr = oracle.quantize_fp4(x)
    k8 = torch.empty((1, n_max, dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((1, n_max), dtype=torch.float32, device=DEV)
    codes = torch.empty((1, n_max, wl.D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((1, wl.D), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf), k8, ks)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(x), codes, scales)
    pos = 2 * Nc + np.arange(T)                                  # token positions of the new rows
    q_limit = ((pos + 1) // 2 - 1).astype(np.int32)[None]
    nk = np.array([n_max], np.int32)
    q, w, qa = wl.index_query(), wl.head_weights(), wl.attn_query()
    ref = oracle.index_score(oracle.PREC_FP8, q, w, k8r, ksr, nk, q_limit=q_limit)
    idx = csa2.index_topk(csa2.PREC_FP8, to_dev(q, torch.bfloat16), to_dev(w), k8, ks, to_dev(nk), wl.K,
                          q_limit=to_dev(q_limit))
    g = idx.cpu().numpy()
    check_topk_near_tie(g, ref, wl.K)
    assert np.all(g <= q_limit[..., None])
    for t in range(T):                                           # entry j's tokens 2j, 2j+1 all <= p
        sel = g[0, t][g[0, t] >= 0]
        assert np.all(2 * sel + 1 <= pos[t])
    out, _ = csa2.sparse_attend(to_dev(qa, torch.bfloat16), codes, scales, idx, wl.softmax_scale,
                                out_dtype=torch.float32)
    ro, _ = oracle.sparse_attend(qa, cr, sr, g, wl.softmax_scale)
    assert max_abs_rel(out.cpu().numpy(), ro) <= 2e-3
