"""GPU parity of multi-token decode in a layer group: T query tokens per sequence (draft
verification; DSpark proposes several tokens at once, "Detailed Notes", DSpark section)
whose own entries are the cache's last T, so token t sees positions below n_keys - (T - 1
- t).  Every row's selection by the near-tie rule on the oracle's scores under that limit
(on the GPU's pool for pooled Reindex rows, whose pool is checked like the single-token
one with the row's visible end), and every row's attention (with its own window) by the
attention bar on the GPU's own selection.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (DEV, build_cache, check_pool, check_pooled_reindex, check_topk_near_tie, max_abs_rel,
                     to_dev)

pytestmark = pytest.mark.gpu

csa2 = pytest.importorskip("compressed_sparse_attention_csa2_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert csa2.device_check() == 0, "not a gfx950 device"


@pytest.mark.parametrize("pool,window", [(None, False), ((8, 64), True)])
def test_multitoken_group(pool, window):
    T = 4
    wl = workloads.workload("group128k", B=3, N=12000, K=128, T=T)
    c = build_cache(wl)
    nk = np.array([12000, 9003, 700], np.int32)
    q_limit = (nk[:, None] - T + np.arange(T)[None, :]).astype(np.int32)
    modes = ["full", "reindex", "reuse", "reindex"]
    rng = np.random.default_rng(5)
    layers, ref_layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        RL = dict(mode=m, q_idx=qi, w=w, q_attn=qa)
        L = dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16))
        if window:
            x = rng.normal(size=(3, 150, wl.D)).astype(np.float32)
            wcr, wsr = oracle.quantize_fp8(x)
            wc = torch.empty((3, 150, wl.D), dtype=torch.uint8, device=DEV)
            wsd = torch.empty((3, 150), dtype=torch.float32, device=DEV)
            csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(x), wc, wsd)
            end = (np.array([[146], [60], [3]]) + np.arange(T)[None, :]).astype(np.int32)
            RL["swa"] = (wcr, wsr, end, 128)
            L["swa"] = csa2.Swa(wc, wsd, to_dev(end), 128)
        if m == "full" and pool:
            L["pool"] = torch.full((3, T, pool[0] * pool[1]), -7, dtype=torch.int32, device=DEV)
        layers.append(L)
        ref_layers.append(RL)
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g_idx = gpool = None
    for i, (L, RL) in enumerate(zip(layers, ref_layers)):
        if L["mode"] == "full" or (L["mode"] == "reindex" and not pool):
            s = oracle.index_score(oracle.PREC_FP8, RL["q_idx"], RL["w"], c["k8_ref"], c["ks_ref"], nk, q_limit=q_limit)
            g_idx = L["idx"].cpu().numpy()
            check_topk_near_tie(g_idx, s, wl.K)
            if pool and L["mode"] == "full":
                gp = L["pool"].cpu().numpy()                      # [B][T][C]
                for t in range(T):
                    check_pool(gp[:, t], s[:, t:t + 1], pool[0], pool[1], q_limit[:, t] + 1)
                gpool = gp
        elif L["mode"] == "reindex":
            g_idx = L["idx"].cpu().numpy()
            for t in range(T):
                check_pooled_reindex(g_idx[:, t:t + 1], RL["q_idx"][:, t:t + 1], RL["w"][:, t:t + 1], c["k8_ref"],
                                     c["ks_ref"], q_limit[:, t] + 1, gpool[:, t], wl.K)
        for b in range(3):
            for t in range(T):
                sel = g_idx[b, t]
                assert np.all(sel[sel >= 0] <= q_limit[b, t]), (i, b, t)
        ro, rl = oracle.sparse_attend(RL["q_attn"], c["codes_ref"], c["scales_ref"], g_idx, wl.softmax_scale,
                                      swa=RL.get("swa"))
        assert max_abs_rel(L["out"].cpu().numpy(), ro) <= 2e-3, i
        assert np.allclose(L["lse"].cpu().numpy(), rl, rtol=2e-3, atol=2e-3), i
