"""Pins of the oracle's multi-token decode in a layer group: T query tokens per sequence
(draft verification: DSpark proposes five tokens at once, "Detailed Notes", DSpark
section) whose own entries are the cache's last T; token t sees positions below
n_keys - (T - 1 - t).

Every row must equal a single-token group run on the cache cut to that row's visible
length (the rule reduces to the T = 1 case), with and without a candidate pool; and the
last row's result must equal the single-token group with the full cache."""
import numpy as np

import oracle
import workloads


def _group(T, nk_b, pool):
    wl = workloads.workload("group128k", B=2, N=3000, K=64, T=T)
    x = np.stack([wl.main_kv(b, rows=3000) for b in range(2)])
    kf = np.stack([wl.index_keys(b, rows=3000) for b in range(2)])
    codes, scales = oracle.quantize_fp4(x)
    k8, ks = oracle.quantize_fp8(kf)
    cache = dict(k=k8, k_scale=ks, n_keys=np.array(nk_b, np.int32), codes=codes, scales=scales)
    layers = [dict(mode=m, q_idx=wl.index_query(i), w=wl.head_weights(i), q_attn=wl.attn_query(i))
              for i, m in enumerate(["full", "reindex", "reuse"])]
    return wl, layers, cache, oracle.layer_group(layers, cache, oracle.PREC_FP8, wl.K, wl.softmax_scale, pool=pool)


def _row(layers, t):
    return [dict(mode=L["mode"], q_idx=L["q_idx"][:, t:t + 1], w=L["w"][:, t:t + 1], q_attn=L["q_attn"][:, t:t + 1])
            for L in layers]


def test_every_row_is_a_single_token_group_on_its_visible_prefix():
    for pool in (None, (8, 32)):
        T, nk = 5, [2990, 1201]
        wl, layers, cache, res = _group(T, nk, pool)
        for t in range(T):
            c1 = dict(cache, n_keys=np.array(nk, np.int32) - (T - 1 - t))
            ref = oracle.layer_group(_row(layers, t), c1, oracle.PREC_FP8, wl.K, wl.softmax_scale, pool=pool)
            for a, b in zip(res, ref):
                assert np.array_equal(a["idx"][:, t:t + 1], b["idx"])
                assert np.array_equal(a["out"][:, t:t + 1], b["out"])
                if "pool" in a:
                    assert np.array_equal(a["pool"][:, t:t + 1], b["pool"])
        # causal: no row selects a position at or past its limit
        for b in range(2):
            for t in range(T):
                sel = res[0]["idx"][b, t]
                assert np.all(sel[sel >= 0] < nk[b] - (T - 1 - t))
