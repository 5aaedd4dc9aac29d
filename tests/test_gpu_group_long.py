"""Layer groups with more Top-K selections than the workspace has histogram slots (64).

Past the 64th selection, the layer group reuses its last slot and clears it again before
each use. Below that, each selection's filter clears the slot the next selection takes. A
long schedule runs through both paths. Every indexing layer's selection must equal, bit for
bit, the standalone csa2_index_score + csa2_topk on the same inputs (same arithmetic, same
strict order). Every layer's output must equal csa2_sparse_attend over the indices the
layer used. The standalone path is pinned to the oracle by the other parity tests.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_csa2_amd as csa2
import workloads
from helpers import DEV, build_cache, to_dev

pytestmark = pytest.mark.gpu


def _layers(wl, modes, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i, m in enumerate(modes):
        j = int(rng.integers(0, 1 << 20))
        out.append(dict(mode=m, q_idx=to_dev(wl.index_query(j), torch.bfloat16), w=to_dev(wl.head_weights(j)),
                        q_attn=to_dev(wl.attn_query(j), torch.bfloat16)))
    return out


@pytest.mark.parametrize("pooled", [False, True])
def test_layer_group_past_the_histogram_slots(pooled):
    wl = workloads.workload("group128k", B=3, N=9000, K=64)
    c = build_cache(wl)
    nk = torch.tensor([9000, 7001, 40], dtype=torch.int32, device=DEV)
    if pooled:
        # a pooled Full layer makes two selections: 34 Full layers give 68
        modes = ["full", "reuse"] * 34
        pool = (8, 64)
    else:
        modes = ["full"] + ["reindex"] * 69  # 70 selections
        pool = None
    print("long group: pooled", pooled, "layers", len(modes), flush=True)
    layers = _layers(wl, modes, 11 if pooled else 12)
    cache = csa2.GroupCache(nk, c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    last = None
    for i, L in enumerate(layers):
        if L["mode"] != "reuse":
            # Full layers scan everything; without a pool, so do the Reindex layers
            s = csa2.index_score(csa2.PREC_FP8, L["q_idx"], L["w"], c["k8"], c["ks"], nk)
            ref = csa2.topk(s, wl.K)
            torch.cuda.synchronize()
            assert torch.equal(L["idx"], ref), i
            last = L["idx"]
        o, lse = csa2.sparse_attend(L["q_attn"], c["codes"], c["scales"], last, wl.softmax_scale,
                                    out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o, L["out"]), i
        assert torch.equal(lse, L["lse"]), i
