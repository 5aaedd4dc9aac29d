"""Pins of the oracle's indexer score and Top-K.

Score: the per-head weighted dot product (reading of "Compressed Sparse Attention 2 Or
CSA2 In Simple Terms": a small per-layer indexer scores past entries) is checked against
torch.einsum in float64 and against its collapsed form.  Top-K ("picks the top 512") is
checked against a brute-force rank count with planted ties.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _brute_topk(scores, K, cand=None):
    # rank_j = #{i : (s_i, -pos_i) > (s_j, -pos_j)} over visible columns; keep rank < K.
    B, T, n = scores.shape
    out = np.full((B, T, K), -1, np.int32)
    for b in range(B):
        for t in range(T):
            s = scores[b, t]
            pos = np.arange(n) if cand is None else cand[b, t]
            vis = [c for c in range(n) if s[c] > -np.inf and pos[c] >= 0]
            chosen = []
            for c in vis:
                rank = sum(1 for i in vis if s[i] > s[c] or (s[i] == s[c] and pos[i] < pos[c]))
                if rank < K:
                    chosen.append(int(pos[c]))
            chosen.sort()
            out[b, t, :len(chosen)] = chosen
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 200))
    K = int(rng.integers(1, 70))
    scores = rng.integers(-5, 6, size=(2, 3, n)).astype(np.float64)   # many planted ties
    scores[rng.random(scores.shape) < 0.1] = -np.inf                  # invisible columns
    assert np.array_equal(oracle.topk(scores, K), _brute_topk(scores, K))


def test_topk_lowest_index_wins_ties():
    scores = np.zeros((1, 1, 10))
    assert list(oracle.topk(scores, 3)[0, 0]) == [0, 1, 2]
    scores[0, 0, 7] = 1.0
    assert list(oracle.topk(scores, 3)[0, 0]) == [0, 1, 7]


def test_topk_more_k_than_visible():
    scores = np.array([[[3.0, -np.inf, 1.0, np.nan, 2.0]]])
    assert list(oracle.topk(scores, 6)[0, 0]) == [0, 2, 4, -1, -1, -1]


def test_topk_with_candidates():
    rng = np.random.default_rng(7)
    cand = rng.permutation(1000)[:300].astype(np.int32).reshape(1, 1, 300)
    cand[0, 0, ::17] = -1
    scores = rng.normal(size=(1, 1, 300))
    got = oracle.topk(scores, 40, cand=cand)
    assert np.array_equal(got, _brute_topk(scores, 40, cand=cand))
    idx, val = oracle.topk(scores, 40, cand=cand, want_values=True)
    m = {int(p): s for p, s in zip(cand[0, 0], scores[0, 0])}
    assert all(val[0, 0, i] == m[int(p)] for i, p in enumerate(idx[0, 0]))


def test_score_fp32_matches_einsum():
    wl = workloads.workload("tiny", N=300)
    q, w = wl.index_query(), wl.head_weights()
    k = wl.index_keys(0)[None]
    n_keys = np.array([300], np.int32)
    s = oracle.index_score(oracle.PREC_FP32, q, w, k, None, n_keys)
    ref = torch.einsum("bthd,bjd,bth->btj", torch.from_numpy(q).double(), torch.from_numpy(k).double(),
                       torch.from_numpy(w).double()).numpy()
    assert np.allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_score_fp8_matches_dequantised_einsum_and_collapsed_form():
    wl = workloads.workload("full64k", N=257, B=2)
    q, w = wl.index_query(), wl.head_weights()
    k = np.stack([wl.index_keys(b) for b in range(wl.B)])
    k8, ks = oracle.quantize_fp8(k)
    n_keys = np.array([257, 200], np.int32)
    s = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, n_keys)
    q8, sq = oracle.quantize_index_query(q)
    f8 = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    kd = f8(k8) * torch.from_numpy(ks).double()[..., None]
    qd = f8(q8) * torch.from_numpy(sq).double()[..., None]
    ref = torch.einsum("bthd,bjd,bth->btj", qd, kd, torch.from_numpy(w).double()).numpy()
    ref[1, :, 200:] = -np.inf
    assert np.array_equal(np.isinf(s), np.isinf(ref))
    fin = np.isfinite(ref)
    assert np.allclose(s[fin], ref[fin], rtol=1e-12, atol=1e-12)
    # collapsed form: (sum_h w_h sq_h q8_h) . k8_j * sk_j
    qeff = torch.einsum("bthd,bth->btd", qd, torch.from_numpy(w).double())
    col = torch.einsum("btd,bjd->btj", qeff, kd).numpy()
    assert np.allclose(s[fin], col[fin], rtol=1e-12, atol=1e-12)


def test_score_visibility_causal_and_candidates():
    wl = workloads.workload("full64k", N=64, T=3, B=1)
    q, w = wl.index_query(), wl.head_weights()
    k8, ks = oracle.quantize_fp8(wl.index_keys(0)[None])
    n_keys = np.array([60], np.int32)
    q_limit = np.array([[10, 59, 63]], np.int32)
    s = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, n_keys, q_limit=q_limit)
    assert np.all(np.isfinite(s[0, 0, :11])) and np.all(np.isinf(s[0, 0, 11:]))
    assert np.all(np.isfinite(s[0, 1, :60])) and np.all(np.isinf(s[0, 1, 60:]))
    assert np.all(np.isfinite(s[0, 2, :60])) and np.all(np.isinf(s[0, 2, 60:]))
    cand = np.array([[[3, -1, 70, 59, 60, 11]] * 3], np.int32)
    sc = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, n_keys, q_limit=q_limit, cand=cand)
    assert sc[0, 0, 0] == s[0, 0, 3] and np.isinf(sc[0, 0, 1]) and np.isinf(sc[0, 0, 2])
    assert np.isinf(sc[0, 0, 3]) and sc[0, 1, 3] == s[0, 1, 59] and np.isinf(sc[0, 2, 4])
    assert np.isinf(sc[0, 0, 5]) and sc[0, 1, 5] == s[0, 1, 11]


def test_causal_prefill_t1_equals_decode():
    # With T = 1 and the query at position N - 1, the causal limit sees exactly what decode sees.
    wl = workloads.workload("full64k", N=128, B=1)
    q, w = wl.index_query(), wl.head_weights()
    k8, ks = oracle.quantize_fp8(wl.index_keys(0)[None])
    nk = np.array([128], np.int32)
    a = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, nk)
    b = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, nk, q_limit=np.array([[127]], np.int32))
    assert np.array_equal(a, b)
    assert np.array_equal(oracle.topk(a, 16), oracle.topk(b, 16))
