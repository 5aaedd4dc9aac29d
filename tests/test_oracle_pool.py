"""Pins of the oracle's candidate pool: a Full layer reduces every block of 8 positions to
its largest score, keeps the best blocks, and later Reindex layers score only the pool's
positions ("Hierarchical Sparse Indexer In Simple Terms")."""
import numpy as np

import oracle
import workloads


def test_block_max_brute_force():
    rng = np.random.default_rng(3)
    s = rng.normal(size=(2, 3, 203))
    s[0, 0, 16:24] = -np.inf                      # a block with nothing visible
    s[1, 2, rng.random(203) < 0.4] = -np.inf
    bm = oracle.block_max(s, 8)
    assert bm.shape == (2, 3, 26)
    for b in range(2):
        for t in range(3):
            for k in range(26):
                seg = s[b, t, 8 * k:8 * k + 8]
                assert bm[b, t, k] == (seg.max() if seg.size else -np.inf)
    assert bm[0, 0, 2] == -np.inf


def test_pool_holds_the_best_blocks_in_ascending_order():
    rng = np.random.default_rng(5)
    n, block, nb_keep = 2000, 8, 40
    s = rng.normal(size=(1, 1, n))
    nk = np.array([1995], np.int32)
    s[..., 1995:] = -np.inf
    pool = oracle.pool_positions(s, block, nb_keep, nk)[0, 0]
    valid = pool[pool >= 0]
    assert np.all(np.diff(valid) > 0) and np.all(valid < 1995)
    bm = oracle.block_max(s, block)[0, 0]
    chosen = np.unique(valid // block)
    assert len(chosen) == nb_keep
    worst_chosen = bm[chosen].min()
    others = np.setdiff1d(np.arange(len(bm)), chosen)
    assert np.all(bm[others] <= worst_chosen)
    # every position of a chosen block that is below n_keys is in the pool
    for blk in chosen:
        assert np.all(np.isin(np.arange(blk * block, min(blk * block + block, 1995)), valid))


def _small_group(pool_blocks, same_query=False):
    wl = workloads.workload("group128k", B=2, N=4096, K=64)
    x = np.stack([wl.main_kv(b, rows=4096) for b in range(2)])
    kf = np.stack([wl.index_keys(b, rows=4096) for b in range(2)])
    codes, scales = oracle.quantize_fp4(x)
    k8, ks = oracle.quantize_fp8(kf)
    cache = dict(k=k8, k_scale=ks, n_keys=np.array([4096, 3001], np.int32), codes=codes, scales=scales)
    layers = []
    for i, m in enumerate(["full", "reindex", "reuse"]):
        li = 0 if same_query else i
        layers.append(dict(mode=m, q_idx=wl.index_query(li), w=wl.head_weights(li), q_attn=wl.attn_query(i)))
    plain = oracle.layer_group(layers, cache, oracle.PREC_FP8, wl.K, wl.softmax_scale)
    pooled = oracle.layer_group(layers, cache, oracle.PREC_FP8, wl.K, wl.softmax_scale, pool=(8, pool_blocks))
    return plain, pooled


def test_pool_covering_every_block_changes_nothing():
    plain, pooled = _small_group(pool_blocks=512)      # 4096 / 8 blocks: the pool is everything
    for a, b in zip(plain, pooled):
        assert np.array_equal(a["idx"], b["idx"])
        assert np.array_equal(a["out"], b["out"])


def test_reindex_with_the_full_query_finds_the_full_selection_inside_the_pool():
    # every Full winner's block has a maximum >= the K-th score, and at most K blocks can,
    # so a pool of >= K blocks holds the whole Full selection
    plain, pooled = _small_group(pool_blocks=64, same_query=True)
    assert np.array_equal(pooled[0]["idx"], pooled[1]["idx"])
    assert np.array_equal(pooled[0]["idx"], plain[0]["idx"])
    pool = pooled[0]["pool"]
    sel = pooled[0]["idx"]
    for b in range(2):
        assert np.all(np.isin(sel[b, 0][sel[b, 0] >= 0], pool[b, 0]))


def test_small_pool_restricts_reindex():
    plain, pooled = _small_group(pool_blocks=16)        # 128 positions: a real restriction
    pool = pooled[0]["pool"]
    for b in range(2):
        got = pooled[1]["idx"][b, 0]
        assert np.all(np.isin(got[got >= 0], pool[b, 0]))
    assert not np.array_equal(plain[1]["idx"], pooled[1]["idx"])
