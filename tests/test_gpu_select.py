"""GPU parity of the decode Top-K on the inputs that defeat the score blocks' candidate
lists, so that the selection must fall back to re-reading whole blocks' scores:

* every key identical: all scores of a row are equal, so every block's cut sits on the one
  bin that holds them all and nothing is listed; the lowest positions must win exactly;
* keys that are one direction scaled by a growing factor: E4M3 per-token quantisation gives
  every key the same codes and a growing scale, so the scores grow with the position and the
  winners are the last K visible positions, all in the last blocks (far more than a block
  lists); with a pool the Reindex selection over the pool falls back the same way;
* rows with only a short visible prefix (every winner in the first blocks).

In the first two cases the scores are exactly ordered (equal, or strictly increasing with
the position), so the expected index sets are exact, not merely within the near-tie band.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_csa2_amd as csa2
import oracle
import workloads
from helpers import DEV, build_cache, check_topk_near_tie, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu


def _keys_device(kf):
    B, n, dk = kf.shape
    k8 = torch.empty((B, n, dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((B, n), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf), k8, ks)
    return k8, ks


def _scaled_direction_keys(B, n, dk=64, seed=5):
    """Keys alpha_j * u: u holds E4M3 values with max |u| = 448 and alpha_j = 1 + j 2^-m
    (exact, strictly increasing, m = bits of n), so each key's scale max|k|/448 is exactly
    alpha_j and its E4M3 codes are exactly u's: every key has the same codes and the scores
    are one product times alpha_j, strictly monotone in j."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, dk)  # finite E4M3 magnitudes
    u = np.array([oracle.e4m3_value(int(cd)) for cd in codes], np.float64)
    u *= np.where(rng.random(dk) < 0.5, -1.0, 1.0)
    u[int(rng.integers(0, dk))] = 448.0
    m = int(np.ceil(np.log2(max(n, 2))))
    alpha = 1.0 + np.arange(n, dtype=np.float64) * 2.0 ** -m
    k = (alpha[:, None] * u[None, :]).astype(np.float32)
    return np.broadcast_to(k[None], (B, n, dk)).copy()


@pytest.mark.parametrize("K", [64, 512, 2048])
def test_index_topk_all_equal_scores_lowest_positions_win(K):
    wl = workloads.workload("group128k", B=2, N=20000, K=K)
    n = wl.N
    kf = np.broadcast_to(wl.index_keys(0, rows=1)[None], (2, n, wl.dk)).astype(np.float32).copy()
    k8, ks = _keys_device(kf)
    nk = np.array([n, 9000], np.int32)
    q, w = wl.index_query(), wl.head_weights()
    s = csa2.index_score(csa2.PREC_FP8, to_dev(q, torch.bfloat16), to_dev(w), k8, ks, to_dev(nk)).cpu().numpy()
    for b in range(2):  # the premise: one score value per row
        assert np.unique(s[b, 0, :nk[b]]).size == 1
    idx = csa2.index_topk(csa2.PREC_FP8, to_dev(q, torch.bfloat16), to_dev(w), k8, ks, to_dev(nk), K)
    g = idx.cpu().numpy()
    for b in range(2):
        assert np.array_equal(g[b, 0], np.arange(K)), b


@pytest.mark.parametrize("K", [64, 512, 1024])
def test_index_topk_scores_growing_with_position_last_positions_win(K):
    wl = workloads.workload("group128k", B=3, N=65536, K=K)
    n = wl.N
    kf = _scaled_direction_keys(3, n)
    k8, ks = _keys_device(kf)
    nk = np.array([n, 40000, 5000], np.int32)
    q, w = wl.index_query(), wl.head_weights()
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    s = csa2.index_score(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk)).cpu().numpy()
    idx = csa2.index_topk(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk), K)
    g = idx.cpu().numpy()
    for b in range(3):
        row = s[b, 0, :nk[b]]
        assert np.all(np.diff(row) > 0) or np.all(np.diff(row) < 0), b  # the premise: strictly monotone
        want = np.arange(nk[b] - K, nk[b]) if row[-1] > row[0] else np.arange(K)
        assert np.array_equal(g[b, 0], want), b
    # the oracle agrees (its scores of the same bytes are ordered the same way)
    k8r, ksr = oracle.quantize_fp8(kf)
    ref = oracle.index_score(oracle.PREC_FP8, q, w, k8r, ksr, nk)
    check_topk_near_tie(g, ref, K)


def test_layer_group_fallback_full_and_pooled_reindex():
    """A pooled group over keys whose scores grow with the position: the Full layer's
    selection and the pool's Reindex selection both fall back; the outputs still match the
    oracle's attention over the same indices."""
    wl = workloads.workload("group128k", B=2, N=30000)
    n = wl.N
    c = build_cache(wl)
    kf = _scaled_direction_keys(2, n)
    k8, ks = _keys_device(kf)
    k8r, ksr = oracle.quantize_fp8(kf)
    nk = np.array([n, 21000], np.int32)
    pool = (8, 512)
    modes = ["full", "reindex", "reuse"]
    layers, ref = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        ref.append(dict(q_idx=qi, w=w, q_attn=qa))
        layers.append(dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16)))
    layers[0]["pool"] = torch.full((2, pool[0] * pool[1]), -7, dtype=torch.int32, device=DEV)
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], k8, ks, wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    s0 = oracle.index_score(oracle.PREC_FP8, ref[0]["q_idx"], ref[0]["w"], k8r, ksr, nk)
    g0 = layers[0]["idx"].cpu().numpy()
    check_topk_near_tie(g0, s0, wl.K)
    for b in range(2):
        row = s0[b, 0, :nk[b]]
        want = np.arange(nk[b] - wl.K, nk[b]) if row[-1] > row[0] else np.arange(wl.K)
        assert np.array_equal(g0[b, 0], want), b
    gp = layers[0]["pool"].cpu().numpy()
    g1 = layers[1]["idx"].cpu().numpy()
    fs = oracle.index_score(oracle.PREC_FP8, ref[1]["q_idx"], ref[1]["w"], k8r, ksr, nk, cand=gp[:, None])
    full = np.full((2, 1, n), -np.inf)
    for b in range(2):
        ok = gp[b] >= 0
        full[b, 0, gp[b][ok]] = fs[b, 0][ok]
        assert np.all(np.isin(g1[b, 0][g1[b, 0] >= 0], gp[b][ok])), b
    check_topk_near_tie(g1, full, wl.K)
    for i, g in [(0, g0), (1, g1), (2, g1)]:
        ro, _ = oracle.sparse_attend(ref[i]["q_attn"], c["codes_ref"], c["scales_ref"], g, wl.softmax_scale)
        out = layers[i]["out"].cpu().numpy()
        for b in range(2):
            assert max_abs_rel(out[b], ro[b]) <= 2e-3, (i, b)


@pytest.mark.parametrize("nk0", [1, 300, 700, 4000])
def test_index_topk_short_visible_prefix(nk0):
    wl = workloads.workload("group128k", B=2, N=65536, K=512)
    c = build_cache(wl)
    nk = np.array([nk0, wl.N], np.int32)
    q, w = wl.index_query(), wl.head_weights()
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    idx = csa2.index_topk(csa2.PREC_FP8, qd, wd, c["k8"], c["ks"], to_dev(nk), wl.K)
    ref = oracle.index_score(oracle.PREC_FP8, q, w, c["k8_ref"], c["ks_ref"], nk)
    check_topk_near_tie(idx.cpu().numpy(), ref, wl.K)


@pytest.mark.parametrize("copies", [300, 1500])
def test_index_topk_many_keys_tied_at_the_top(copies):
    """The best key of each row copied to `copies` further random positions: that many keys
    share the largest score (same codes, same scale), spread over the score blocks so that
    each block lists its share.  With 1500 copies more than a thousand listed candidates hold
    one key value, the selection's equal-key branch; the K winners are then the lowest
    positions among the tied keys, exactly."""
    wl = workloads.workload("group128k", B=2, N=131072, K=512)
    n = wl.N
    rng = np.random.default_rng(31)
    kf = np.stack([wl.index_keys(b) for b in range(2)])
    q, w = wl.index_query(), wl.head_weights()
    k8r, ksr = oracle.quantize_fp8(kf)
    nk = np.array([n, 100000], np.int32)
    ref = oracle.index_score(oracle.PREC_FP8, q, w, k8r, ksr, nk)
    for b in range(2):
        best = int(np.argmax(ref[b, 0, :nk[b]]))
        dst = rng.choice(nk[b], size=copies, replace=False)
        kf[b, dst] = kf[b, best]
    k8, ks = _keys_device(kf)
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    s = csa2.index_score(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk)).cpu().numpy()
    g = csa2.index_topk(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk), wl.K).cpu().numpy()
    for b in range(2):
        row = s[b, 0, :nk[b]]
        tied = np.flatnonzero(row == row.max())
        assert tied.size >= copies + 1, b  # the premise: the copies tie with the best key
        if tied.size >= wl.K:  # the lowest positions among the tied keys, exactly
            assert np.array_equal(g[b, 0], tied[:wl.K]), b
        else:                  # every tied key wins
            assert np.all(np.isin(tied, g[b, 0])), b
    k8r2, ksr2 = oracle.quantize_fp8(kf)
    check_topk_near_tie(g, oracle.index_score(oracle.PREC_FP8, q, w, k8r2, ksr2, nk), wl.K)


@pytest.mark.parametrize("kind", ["equal", "growing"])
def test_many_row_topk_fallback(kind):
    """The many-row (chunked prefill) selection on keys that defeat its candidate lists:
    every score equal (nothing is listed; the lowest positions win) or scores growing with
    the position (the winners are each row's last K visible positions, more than a region
    lists).  16 rows with causal limits, so that rows see different prefixes."""
    K = 512
    wl = workloads.workload("prefill", N=20000, T=16, K=K)
    n = wl.N + wl.T
    if kind == "equal":
        kf = np.broadcast_to(wl.index_keys(0, rows=1)[None], (1, n, wl.dk)).astype(np.float32).copy()
    else:
        kf = _scaled_direction_keys(1, n)
    k8, ks = _keys_device(kf)
    nk = np.array([n], np.int32)
    ql = (wl.N + np.arange(wl.T, dtype=np.int32))[None]
    q, w = wl.index_query(), wl.head_weights()
    qd, wd = to_dev(q, torch.bfloat16), to_dev(w)
    s = csa2.index_score(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk), q_limit=to_dev(ql)).cpu().numpy()
    g = csa2.index_topk(csa2.PREC_FP8, qd, wd, k8, ks, to_dev(nk), K, q_limit=to_dev(ql)).cpu().numpy()
    for t in range(wl.T):
        row = s[0, t, :ql[0, t] + 1]
        if kind == "equal":
            assert np.unique(row).size == 1, t
            want = np.arange(K)
        else:
            assert np.all(np.diff(row) > 0) or np.all(np.diff(row) < 0), t
            want = np.arange(ql[0, t] + 1 - K, ql[0, t] + 1) if row[-1] > row[0] else np.arange(K)
        assert np.array_equal(g[0, t], want), t
    k8r, ksr = oracle.quantize_fp8(kf)
    check_topk_near_tie(g, oracle.index_score(oracle.PREC_FP8, q, w, k8r, ksr, nk, q_limit=ql), K)
