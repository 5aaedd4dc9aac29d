"""csa2_layer_group_noalloc (the layer group whose workspace is the library's own scratch
array) against csa2_layer_group with a caller workspace: two calls in a row, the second
on a smaller input, each bit-identical to the workspace entry point on the same inputs
(same kernels, deterministic), and within the oracle's bars."""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_csa2_amd as csa2
import oracle
import workloads
from helpers import DEV, build_cache, check_topk_near_tie, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu


def _layers(wl, modes, seed_off):
    layers, ref = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i + seed_off), wl.head_weights(i + seed_off), wl.attn_query(i + seed_off)
        ref.append(dict(mode=m, q_idx=qi, w=w, q_attn=qa))
        layers.append(dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16)))
    return layers, ref


def _copy_inputs(layers):
    return [{k: v for k, v in L.items() if k in ("mode", "q_idx", "w", "q_attn")} for L in layers]


def _run_both(wl, c, nk, modes, seed_off):
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale)
    a, ref = _layers(wl, modes, seed_off)
    b = _copy_inputs(a)
    csa2.layer_group_noalloc(a, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    csa2.layer_group(b, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx_last = None
    for i, (La, Lb) in enumerate(zip(a, b)):
        assert torch.equal(La["out"], Lb["out"]) and torch.equal(La["lse"], Lb["lse"]), i
        if La["mode"] != "reuse":
            assert torch.equal(La["idx"], Lb["idx"]), i
            s = oracle.index_score(oracle.PREC_FP8, ref[i]["q_idx"], ref[i]["w"], c["k8_ref"], c["ks_ref"], nk)
            idx_last = La["idx"].cpu().numpy()
            check_topk_near_tie(idx_last, s, wl.K)
        ro, _ = oracle.sparse_attend(ref[i]["q_attn"], c["codes_ref"], c["scales_ref"], idx_last, wl.softmax_scale)
        out = La["out"].cpu().numpy()
        for bb in range(len(nk)):
            assert max_abs_rel(out[bb], ro[bb]) <= 2e-3, (i, bb)


def test_noalloc_matches_workspace_entry_point_two_calls():
    wl = workloads.workload("group128k", B=3, N=12000)
    c = build_cache(wl)
    _run_both(wl, c, np.array([12000, 9000, 3000], np.int32), ["full", "reindex", "reuse"], 0)
    # second call: a smaller input (fewer sequences, shorter cache, one layer less)
    wl2 = workloads.workload("group128k", B=2, N=5000)
    c2 = build_cache(wl2)
    _run_both(wl2, c2, np.array([5000, 4100], np.int32), ["full", "reuse"], 7)
