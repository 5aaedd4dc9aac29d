"""GPU parity at the full sizes of the measured configurations, in the launch
configuration bench.py times.

The whole batch runs on the GPU. The oracle recomputes a sample of sequences (or query
rows) one by one: the cache bytes of the sampled sequences bit-exact, the Top-K sets
under the near-tie rule, and the attention outputs under the bf16 rule. A second run of
the same call must reproduce every output bit.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_csa2_amd as csa2
import oracle
import workloads
from helpers import DEV, check_pool, check_pooled_reindex, check_topk_near_tie, to_dev

pytestmark = pytest.mark.gpu


def _bf16_ok(out, ref):
    """bf16-written output: per element within 2e-3 * max|ref| plus half a bf16 ulp."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return bool(np.all(np.abs(out - ref) <= 2e-3 * np.abs(ref).max() + np.abs(ref) * 2.0 ** -8))


def _device_cache_with_samples(wl, sample):
    """Quantise every sequence on the GPU, one at a time, as bench.py does; the sampled
    sequences are also quantised by the oracle and compared byte for byte."""
    B, N, D, dk = wl.B, wl.N, wl.D, wl.dk
    codes = torch.empty((B, N, D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, D), dtype=torch.float32, device=DEV)
    k8 = torch.empty((B, N, dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((B, N), dtype=torch.float32, device=DEV)
    ref = {}
    for b in range(B):
        x = wl.main_kv(b)
        kf = wl.index_keys(b)
        csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(x)[None], codes[b:b + 1], scales[b:b + 1])
        csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf)[None], k8[b:b + 1], ks[b:b + 1])
        if b in sample:
            cr, sr = oracle.quantize_fp4(x[None])
            kr, ksr = oracle.quantize_fp8(kf[None])
            torch.cuda.synchronize()
            assert np.array_equal(codes[b].cpu().numpy(), cr[0]), b
            assert np.array_equal(scales[b].cpu().numpy(), sr[0]), b
            assert np.array_equal(k8[b].cpu().numpy(), kr[0]), b
            assert np.array_equal(ks[b].cpu().numpy(), ksr[0]), b
            ref[b] = (cr[0], sr[0], kr[0], ksr[0])
    torch.cuda.synchronize()
    return dict(codes=codes, scales=scales, k8=k8, ks=ks), ref


def _check_group_against_oracle(wl, modes, dev_layers, ref_cache, sample, q_in):
    """Every layer of the sampled sequences: an indexing layer's selection by the near-tie
    rule on the oracle's scores; every layer's output and log-sum-exp against the oracle's
    attention over the index tensor the GPU layer attended (its own selection, or for
    Reuse the last indexing layer's), so the outputs are always compared."""
    idx_last = None
    checked = 0
    for i, (L, m) in enumerate(zip(dev_layers, modes)):
        qi, w, qa = (x[sample] for x in q_in[i])
        if m != "reuse":
            s = oracle.index_score(oracle.PREC_FP8, qi, w, ref_cache["k"], ref_cache["k_scale"], ref_cache["n_keys"])
            idx_last = L["idx"].cpu().numpy()[sample]
            check_topk_near_tie(idx_last, s, wl.K)
        ro, rl = oracle.sparse_attend(qa, ref_cache["codes"], ref_cache["scales"], idx_last, wl.softmax_scale)
        out = L["out"].float().cpu().numpy()[sample]
        lse = L["lse"].cpu().numpy()[sample]
        for j in range(len(sample)):
            assert _bf16_ok(out[j], ro[j]), (i, sample[j])
            assert np.allclose(lse[j], rl[j], rtol=0, atol=2e-3 * max(1.0, np.abs(rl[j]).max())), (i, sample[j])
            checked += 1
    assert checked == len(modes) * len(sample)
    return checked


def test_group128k_full_size_sampled_sequences():
    """The 128K decode configuration: Full -> Reindex -> Reuse, 16 sequences x 131072."""
    wl = workloads.WORKLOADS["group128k"]
    sample = [0, 9, 15]
    c, ref = _device_cache_with_samples(wl, sample)
    n_keys = torch.full((wl.B,), wl.N, dtype=torch.int32, device=DEV)
    q_in, layers = [], []
    for i, m in enumerate(wl.modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        q_in.append((qi, w, qa))
        layers.append(dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16)))
    cache = csa2.GroupCache(n_keys, c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale)
    plan = csa2.GroupPlan(layers, cache, out_dtype=torch.bfloat16)
    plan.run()
    torch.cuda.synchronize()
    first = [(L["out"].clone(), L["lse"].clone(), L.get("idx").clone() if L.get("idx") is not None else None)
             for L in layers]
    ref_cache = dict(k=np.stack([ref[b][2] for b in sample]), k_scale=np.stack([ref[b][3] for b in sample]),
                     n_keys=np.full(len(sample), wl.N, np.int32), codes=np.stack([ref[b][0] for b in sample]),
                     scales=np.stack([ref[b][1] for b in sample]))
    _check_group_against_oracle(wl, wl.modes, layers, ref_cache, sample, q_in)
    # determinism: the same call again gives the same bits
    plan.run()
    torch.cuda.synchronize()
    for L, (o, l, ix) in zip(layers, first):
        assert torch.equal(L["out"], o) and torch.equal(L["lse"], l)
        if ix is not None:
            assert torch.equal(L["idx"], ix)


def test_decoder128k_pool_full_size_sampled_sequences():
    """The 128K decode configuration with the candidate pool of the pages' decoder: the Full
    layer keeps its best 2048 blocks of 8 (16384 positions) and the Reindex layers score only
    those.  16 sequences x 131072, schedule Full, Reuse, Reindex, Reuse, Reindex."""
    wl = workloads.WORKLOADS["group128k"]
    sample = [0, 9, 15]
    pool = (8, 2048)
    modes = ["full", "reuse", "reindex", "reuse", "reindex"]
    c, ref = _device_cache_with_samples(wl, sample)
    n_keys = torch.full((wl.B,), wl.N, dtype=torch.int32, device=DEV)
    q_in, layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        q_in.append((qi, w, qa))
        L = dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16))
        if m == "full":
            L["pool"] = torch.full((wl.B, pool[0] * pool[1]), -7, dtype=torch.int32, device=DEV)
        layers.append(L)
    cache = csa2.GroupCache(n_keys, c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale, pool=pool)
    plan = csa2.GroupPlan(layers, cache, out_dtype=torch.bfloat16)
    plan.run()
    torch.cuda.synchronize()
    first = [L["out"].clone() for L in layers]
    k8 = np.stack([ref[b][2] for b in sample])
    ks = np.stack([ref[b][3] for b in sample])
    codes = np.stack([ref[b][0] for b in sample])
    scales = np.stack([ref[b][1] for b in sample])
    nk = np.full(len(sample), wl.N, np.int32)
    gpool = g_idx = None
    for i, (L, m) in enumerate(zip(layers, modes)):
        qi, w, qa = (x[sample] for x in q_in[i])
        if m == "full":
            s = oracle.index_score(oracle.PREC_FP8, qi, w, k8, ks, nk)
            g_idx = L["idx"].cpu().numpy()[sample]
            check_topk_near_tie(g_idx, s, wl.K)
            gpool = L["pool"].cpu().numpy()[sample]
            check_pool(gpool, s, pool[0], pool[1], nk)
            assert np.all(gpool >= 0)  # 16384 blocks to choose 2048 from: every slot filled
        elif m == "reindex":
            g_idx = L["idx"].cpu().numpy()[sample]
            check_pooled_reindex(g_idx, qi, w, k8, ks, nk, gpool, wl.K)
        ro, _ = oracle.sparse_attend(qa, codes, scales, g_idx, wl.softmax_scale)
        assert _bf16_ok(L["out"].float().cpu().numpy()[sample], ro), i
    plan.run()
    torch.cuda.synchronize()
    for L, o in zip(layers, first):
        assert torch.equal(L["out"], o)


def test_group128k_g16_full_size_sampled_sequences():
    """The 128K decode group with the pages' FP4 layout (one E4M3 scale per 16 channels of
    each entry, 288 B per entry): Full -> Reindex -> Reuse, 16 sequences x 131072."""
    wl = workloads.WORKLOADS["group128k"]
    sample = [2, 13]
    B, N, D, dk = wl.B, wl.N, wl.D, wl.dk
    codes = torch.empty((B, N, D // 2), dtype=torch.uint8, device=DEV)
    gs = torch.empty((B, N, D // 16), dtype=torch.uint8, device=DEV)
    k8 = torch.empty((B, N, dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((B, N), dtype=torch.float32, device=DEV)
    ref = {}
    for b in range(B):
        x, kf = wl.main_kv(b), wl.index_keys(b)
        csa2.quantize_kv(csa2.FMT_FP4_G16, to_dev(x)[None], codes[b:b + 1], gs[b:b + 1])
        csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf)[None], k8[b:b + 1], ks[b:b + 1])
        if b in sample:
            cr, gr = oracle.quantize_fp4_g16(x[None])
            kr, ksr = oracle.quantize_fp8(kf[None])
            torch.cuda.synchronize()
            assert np.array_equal(codes[b].cpu().numpy(), cr[0]) and np.array_equal(gs[b].cpu().numpy(), gr[0]), b
            assert np.array_equal(k8[b].cpu().numpy(), kr[0]) and np.array_equal(ks[b].cpu().numpy(), ksr[0]), b
            ref[b] = (cr[0], gr[0], kr[0], ksr[0])
    n_keys = torch.full((B,), N, dtype=torch.int32, device=DEV)
    q_in, layers = [], []
    for i, m in enumerate(wl.modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        q_in.append((qi, w, qa))
        layers.append(dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16)))
    cache = csa2.GroupCache(n_keys, codes, gs, k8, ks, wl.K, wl.softmax_scale)
    csa2.layer_group(layers, cache, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cr = np.stack([ref[b][0] for b in sample])
    gr = np.stack([ref[b][1] for b in sample])
    kr = np.stack([ref[b][2] for b in sample])
    ksr = np.stack([ref[b][3] for b in sample])
    nk = np.full(len(sample), N, np.int32)
    g_idx = None
    for i, (L, m) in enumerate(zip(layers, wl.modes)):
        qi, w, qa = (x[sample] for x in q_in[i])
        if m != "reuse":
            s = oracle.index_score(oracle.PREC_FP8, qi, w, kr, ksr, nk)
            g_idx = L["idx"].cpu().numpy()[sample]
            check_topk_near_tie(g_idx, s, wl.K)
        ro, _ = oracle.sparse_attend(qa, cr, gr, g_idx, wl.softmax_scale)
        assert _bf16_ok(L["out"].float().cpu().numpy()[sample], ro), i


def test_full64k_full_size_sampled_sequences():
    """The single-layer 64K decode configuration: Full, 16 sequences x 65536."""
    wl = workloads.WORKLOADS["full64k"]
    sample = [3, 12]
    c, ref = _device_cache_with_samples(wl, sample)
    n_keys = torch.full((wl.B,), wl.N, dtype=torch.int32, device=DEV)
    qi, w, qa = wl.index_query(0), wl.head_weights(0), wl.attn_query(0)
    layers = [dict(mode="full", q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16))]
    cache = csa2.GroupCache(n_keys, c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale)
    csa2.layer_group(layers, cache, out_dtype=torch.bfloat16)
    ref_cache = dict(k=np.stack([ref[b][2] for b in sample]), k_scale=np.stack([ref[b][3] for b in sample]),
                     n_keys=np.full(len(sample), wl.N, np.int32), codes=np.stack([ref[b][0] for b in sample]),
                     scales=np.stack([ref[b][1] for b in sample]))
    _check_group_against_oracle(wl, ["full"], layers, ref_cache, sample, [(qi, w, qa)])


def test_hier1m_full_size():
    """The 1M-entry two-level configuration: coarse keys of 64-entry blocks, top-256 blocks,
    Top-1024 inside them, then attention over the 1024 entries (two splits merged)."""
    wl = workloads.WORKLOADS["hier1m"]
    n = wl.N
    x = wl.main_kv(0)
    kf = wl.index_keys(0)
    kr, ksr = oracle.quantize_fp8(kf[None])
    nk = np.array([n], np.int32)
    kb_ref, kbs_ref = oracle.coarse_keys(kr, ksr, nk, wl.coarse_block)
    k8 = torch.empty((1, n, wl.dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((1, n), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf)[None], k8, ks)
    codes = torch.empty((1, n, wl.D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((1, wl.D), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(x)[None], codes, scales)
    kb, kbs = csa2.coarse_keys(k8, ks, to_dev(nk), wl.coarse_block)
    assert np.array_equal(kb.cpu().numpy(), kb_ref) and np.array_equal(kbs.cpu().numpy(), kbs_ref)
    q, w = wl.index_query(), wl.head_weights()
    idx, blk = csa2.hier_select(to_dev(q, torch.bfloat16), to_dev(w), k8, ks, kb, kbs, to_dev(nk), wl.coarse_block,
                                wl.coarse_topk, wl.K, want_blocks=True)
    cs = oracle.index_score(oracle.PREC_FP8, q, w, kb_ref, kbs_ref, (nk + wl.coarse_block - 1) // wl.coarse_block)
    check_topk_near_tie(blk.cpu().numpy(), cs, wl.coarse_topk)
    g_idx = idx.cpu().numpy()
    # the fine stage on the GPU's own block list (whatever blocks it kept within the near-tie
    # band): near-tie rule on the oracle's scores of exactly those candidates, all inside them
    cand = oracle.expand_blocks(blk.cpu().numpy(), wl.coarse_block, nk)
    fs = oracle.index_score(oracle.PREC_FP8, q, w, kr, ksr, nk, cand=cand)
    full = np.full((1, 1, n), -np.inf)
    c0 = cand[0, 0]
    full[0, 0, c0[c0 >= 0]] = fs[0, 0][c0 >= 0]
    check_topk_near_tie(g_idx, full, wl.K)
    assert np.all(np.isin(g_idx[g_idx >= 0], c0[c0 >= 0]))
    # attention over the GPU's selection on both sides
    qa = wl.attn_query()
    cr, sr = oracle.quantize_fp4(x[None])
    assert np.array_equal(codes.cpu().numpy(), cr)
    out, lse = csa2.sparse_attend(to_dev(qa, torch.bfloat16), codes, scales, idx, wl.softmax_scale,
                                  out_dtype=torch.bfloat16)
    ro, rl = oracle.sparse_attend(qa, cr, sr, g_idx, wl.softmax_scale)
    assert _bf16_ok(out.float().cpu().numpy(), ro)
    assert np.allclose(lse.cpu().numpy(), rl, rtol=0, atol=2e-3 * max(1.0, np.abs(rl).max()))


def test_hier_step_graph_replay_matches_eager():
    """The two-level select + attention captured into a HIP graph: every replay (with eager
    work and synchronisation between replays) reproduces the eager result bit for bit."""
    wl = workloads.workload("hier1m", N=64 * 4096)
    n = wl.N
    k8 = torch.empty((1, n, wl.dk), dtype=torch.uint8, device=DEV)
    ks = torch.empty((1, n), dtype=torch.float32, device=DEV)
    codes = torch.empty((1, n, wl.D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((1, wl.D), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(wl.index_keys(0))[None], k8, ks)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, to_dev(wl.main_kv(0))[None], codes, scales)
    nk = torch.tensor([n - 77], dtype=torch.int32, device=DEV)
    kb, kbs = csa2.coarse_keys(k8, ks, nk, wl.coarse_block)
    q = to_dev(wl.index_query(), torch.bfloat16)
    w = to_dev(wl.head_weights())
    qa = to_dev(wl.attn_query(), torch.bfloat16)
    out = torch.empty((1, 1, wl.Hq, wl.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, 1, wl.Hq), dtype=torch.float32, device=DEV)
    holder = {}

    def step():
        holder["idx"] = csa2.hier_select(q, w, k8, ks, kb, kbs, nk, wl.coarse_block, wl.coarse_topk, wl.K)
        csa2.sparse_attend(qa, codes, scales, holder["idx"], wl.softmax_scale, out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = (holder["idx"].clone(), out.clone(), lse.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    g_idx = holder["idx"]  # the index tensor the graph writes
    for rep in range(4):
        out.zero_()
        lse.zero_()
        g_idx.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_idx, ref[0]), rep
        assert torch.equal(out, ref[1]) and torch.equal(lse, ref[2]), rep
        step()  # eager work between replays
        torch.cuda.synchronize()
