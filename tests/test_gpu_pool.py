"""GPU parity of the candidate pool ("Hierarchical Sparse Indexer In Simple Terms", Figure 5):
a Full layer reduces its scores over blocks of `block` consecutive positions to the block
maximum, keeps the best `blocks` blocks and expands them to positions; the Reindex layers
after it score only that pool.

Checks, each against the oracle on the same cache bytes:
* the pool: its block list passes the near-tie rule on the oracle's block maxima, and the
  positions are exactly the expansion of that block list;
* every Reindex selection passes the near-tie rule on the oracle's scores restricted to the
  GPU's pool (the pool of the most recent Full layer), every Full selection on the full scan;
* every layer's output agrees with the oracle's attention over the GPU's own selection
  (2e-3 max-abs-relative on the bf16 path, 1e-5 on the fp32 path).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import DEV, build_cache, check_pool, check_pooled_reindex, check_topk_near_tie, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu

csa2 = pytest.importorskip("compressed_sparse_attention_csa2_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert csa2.device_check() == 0, "not a gfx950 device"


def run_group(wl, c, nk, modes, pool, q_dtype):
    B = len(nk)
    C = pool[0] * pool[1]
    layers, ref_layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        ref_layers.append(dict(mode=m, q_idx=qi, w=w, q_attn=qa))
        L = dict(mode=m, q_idx=to_dev(qi, q_dtype), w=to_dev(w), q_attn=to_dev(qa, q_dtype))
        if m == "full":
            L["pool"] = torch.full((B, C), -7, dtype=torch.int32, device=DEV)
        layers.append(L)
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return layers, ref_layers


def check_group(wl, c, nk, layers, ref_layers, pool, tol):
    gpool, g_idx = None, None
    for i, (L, RL) in enumerate(zip(layers, ref_layers)):
        if L["mode"] == "full":
            s = oracle.index_score(oracle.PREC_FP8, RL["q_idx"], RL["w"], c["k8_ref"], c["ks_ref"], nk)
            g_idx = L["idx"].cpu().numpy()
            check_topk_near_tie(g_idx, s, wl.K)
            gpool = L["pool"].cpu().numpy()
            check_pool(gpool, s, pool[0], pool[1], nk)
        elif L["mode"] == "reindex":
            g_idx = L["idx"].cpu().numpy()
            check_pooled_reindex(g_idx, RL["q_idx"], RL["w"], c["k8_ref"], c["ks_ref"], nk, gpool, wl.K)
        ro, _ = oracle.sparse_attend(RL["q_attn"], c["codes_ref"], c["scales_ref"], g_idx, wl.softmax_scale)
        assert max_abs_rel(L["out"].cpu().numpy(), ro) <= tol, i


@pytest.mark.parametrize("q_dtype,tol", [(torch.bfloat16, 2e-3), (torch.float32, 1e-5)])
def test_pool_group_small(q_dtype, tol):
    """Two Full layers, each followed by Reindex layers that must use the newer pool; one
    sequence (700 keys, 88 blocks) has fewer visible blocks than the pool holds."""
    wl = workloads.workload("group128k", B=3, N=20000, K=256)
    c = build_cache(wl)
    nk = np.array([20000, 19003, 700], np.int32)
    modes = ["full", "reindex", "reuse", "full", "reindex", "reindex", "reuse"]
    pool = (8, 128)
    layers, ref_layers = run_group(wl, c, nk, modes, pool, q_dtype)
    check_group(wl, c, nk, layers, ref_layers, pool, tol)
    short = layers[0]["pool"].cpu().numpy()[2]
    assert np.all(short[88 * 8:] == -1) and np.all(short[:700] == np.arange(700))


def test_pool_wider_than_the_cache_is_the_full_scan():
    """blocks of 16 x 2048 blocks = 32768 positions > 20000 keys: the pool is every visible
    position, so the Reindex layer's selection passes the rule on the full scan too."""
    wl = workloads.workload("group128k", B=2, N=20000)
    c = build_cache(wl)
    nk = np.array([20000, 12345], np.int32)
    pool = (16, 2048)
    layers, ref_layers = run_group(wl, c, nk, ["full", "reindex", "reuse"], pool, torch.bfloat16)
    check_group(wl, c, nk, layers, ref_layers, pool, 2e-3)
    gp = layers[0]["pool"].cpu().numpy()
    for b in range(2):
        assert np.array_equal(gp[b][:nk[b]], np.arange(nk[b])) and np.all(gp[b][nk[b]:] == -1)
    s = oracle.index_score(oracle.PREC_FP8, ref_layers[1]["q_idx"], ref_layers[1]["w"], c["k8_ref"], c["ks_ref"], nk)
    check_topk_near_tie(layers[1]["idx"].cpu().numpy(), s, wl.K)
