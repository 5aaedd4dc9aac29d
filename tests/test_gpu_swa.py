"""GPU parity of the sliding-window part of the attention: every layer also attends to its
own most recent entries, in the same softmax as its selected entries ("CSA2 In Simple
Terms"; window 128 in "Model Setup Numbers"; the window cache stays 8-bit in "FP4 Main KV
Cache To Halve Storage Again").

The window cache is E4M3 with one fp32 scale per row, written by the library and checked
byte-exact against the oracle.  Attention bars as for the selection alone: 2e-3 max-abs-
relative on the bf16 MFMA path (fp32 output), bf16 output within 2e-3 * max|ref| plus half
a bf16 ulp, 1e-5 on the fp32 path; lse within 2e-3 (1e-5).  Windows cover the full, short,
empty and clamped cases; layer groups give every layer its own window.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import DEV, build_cache, check_topk_near_tie, max_abs_rel, to_dev

pytestmark = pytest.mark.gpu

csa2 = pytest.importorskip("compressed_sparse_attention_csa2_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert csa2.device_check() == 0, "not a gfx950 device"


def window_cache(B, n, D, seed):
    """A layer's window cache: N(0,1) rows (a few large channels) quantised to E4M3 per row
    on both sides, bytes checked equal."""
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(B, n, D)).astype(np.float32)
    x[:, :, rng.choice(D, 4, replace=False)] *= 8.0
    cr, sr = oracle.quantize_fp8(x)
    codes = torch.empty((B, n, D), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, n), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(x), codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), cr) and np.array_equal(scales.cpu().numpy(), sr)
    return codes, scales, cr, sr


@pytest.mark.parametrize("K,D", [(512, 512), (100, 512), (1024, 512), (512, 256), (300, 128)])
def test_sparse_attend_with_window_bf16(K, D):
    B = 4
    wl = workloads.workload("full64k", B=B, K=K, D=D)
    c = build_cache(wl, n_rows=3000)
    q = wl.attn_query()
    rng = np.random.default_rng(K + D)
    idx = np.stack([np.sort(rng.choice(3000, K, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    idx[1, 0, ::3] = -1
    wc, ws, wcr, wsr = window_cache(B, 200, D, seed=K)
    end = np.array([[200], [5], [0], [777]], np.int32)   # full, short, empty, past the cache end
    ref_o, ref_l = oracle.sparse_attend(q, c["codes_ref"], c["scales_ref"], idx, wl.softmax_scale,
                                        swa=(wcr, wsr, end, 128))
    sw = csa2.Swa(wc, ws, to_dev(end), 128)
    qd = to_dev(q, torch.bfloat16)
    out, lse = csa2.sparse_attend(qd, c["codes"], c["scales"], to_dev(idx), wl.softmax_scale,
                                  out_dtype=torch.float32, swa=sw)
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)
    ob, _ = csa2.sparse_attend(qd, c["codes"], c["scales"], to_dev(idx), wl.softmax_scale,
                               out_dtype=torch.bfloat16, swa=sw)
    ob = ob.float().cpu().numpy()
    assert np.all(np.abs(ob - ref_o) <= 2e-3 * np.abs(ref_o).max() + np.abs(ref_o) * 2.0 ** -8)


def test_window_only_and_nothing_at_all():
    wl = workloads.workload("full64k", B=2, K=512)
    c = build_cache(wl, n_rows=600)
    q = wl.attn_query()
    idx = np.full((2, 1, 512), -1, np.int32)
    wc, ws, wcr, wsr = window_cache(2, 130, 512, seed=1)
    end = np.array([[130], [0]], np.int32)
    ref_o, ref_l = oracle.sparse_attend(q, c["codes_ref"], c["scales_ref"], idx, wl.softmax_scale,
                                        swa=(wcr, wsr, end, 100))
    out, lse = csa2.sparse_attend(to_dev(q, torch.bfloat16), c["codes"], c["scales"], to_dev(idx), wl.softmax_scale,
                                  out_dtype=torch.float32, swa=csa2.Swa(wc, ws, to_dev(end), 100))
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert max_abs_rel(o[0], ref_o[0]) <= 2e-3 and np.allclose(l[0], ref_l[0], rtol=2e-3, atol=2e-3)
    assert np.all(o[1] == 0) and np.all(np.isneginf(l[1]))


def test_window_with_g16_cache_and_fp32_path():
    wl = workloads.WORKLOADS["tiny"]                      # fp32 queries, D = 128, 8 heads
    x = wl.main_kv(0)[None]
    cr, gr = oracle.quantize_fp4_g16(x)
    codes = torch.empty((1, wl.N, 64), dtype=torch.uint8, device=DEV)
    gs = torch.empty((1, wl.N, 8), dtype=torch.uint8, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_G16, to_dev(x), codes, gs)
    q = wl.attn_query()
    rng = np.random.default_rng(2)
    idx = np.sort(rng.choice(wl.N, 64, replace=False)).astype(np.int32)[None, None]
    idx[0, 0, -3:] = -1
    wc, ws, wcr, wsr = window_cache(1, 150, 128, seed=4)
    end = np.array([[140]], np.int32)
    ref_o, ref_l = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale, swa=(wcr, wsr, end, 128))
    out, lse = csa2.sparse_attend(to_dev(q), codes, gs, to_dev(idx), wl.softmax_scale,
                                  swa=csa2.Swa(wc, ws, to_dev(end), 128))
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 1e-5
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=1e-5, atol=1e-5)
    # the same with bf16 queries and 16 heads on the MFMA path
    wl2 = workloads.workload("full64k", B=1, K=64, D=128, Hq=16)
    q2 = wl2.attn_query()
    ref_o, ref_l = oracle.sparse_attend(q2, cr, gr, idx, wl2.softmax_scale, swa=(wcr, wsr, end, 128))
    out, lse = csa2.sparse_attend(to_dev(q2, torch.bfloat16), codes, gs, to_dev(idx), wl2.softmax_scale,
                                  out_dtype=torch.float32, swa=csa2.Swa(wc, ws, to_dev(end), 128))
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("pool", [None, (8, 128)])
def test_layer_group_with_a_window_per_layer(pool):
    wl = workloads.workload("group128k", B=3, N=20000, K=256)
    c = build_cache(wl)
    nk = np.array([20000, 15001, 900], np.int32)
    modes = ["full", "reuse", "reindex", "reuse"]
    layers, ref_layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        wc, ws, wcr, wsr = window_cache(3, 140, wl.D, seed=10 + i)     # every layer its own window cache
        end = np.array([[140], [64 + i], [0 if i == 1 else 3]], np.int32)
        ref_layers.append(dict(mode=m, q_idx=qi, w=w, q_attn=qa, swa=(wcr, wsr, end, 128)))
        layers.append(dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16),
                           swa=csa2.Swa(wc, ws, to_dev(end), 128)))
    cache = csa2.GroupCache(to_dev(nk), c["codes"], c["scales"], c["k8"], c["ks"], wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g_idx = None
    for i, (L, RL) in enumerate(zip(layers, ref_layers)):
        if L["mode"] != "reuse":
            g_idx = L["idx"].cpu().numpy()
            if L["mode"] == "full" or pool is None:
                s = oracle.index_score(oracle.PREC_FP8, RL["q_idx"], RL["w"], c["k8_ref"], c["ks_ref"], nk)
                check_topk_near_tie(g_idx, s, wl.K)
        ro, rl = oracle.sparse_attend(RL["q_attn"], c["codes_ref"], c["scales_ref"], g_idx, wl.softmax_scale,
                                      swa=RL["swa"])
        assert max_abs_rel(L["out"].cpu().numpy(), ro) <= 2e-3, i
        assert np.allclose(L["lse"].cpu().numpy(), rl, rtol=2e-3, atol=2e-3), i


def test_sparse_attend_with_window_many_rows():
    """72 rows: more attention blocks than fit one round on the chip, where the window runs as a
    block column of its own and its partial is merged with the selection's (the decode shapes
    attend it inside the selection's blocks instead)."""
    B = 72
    wl = workloads.workload("full64k", B=B, K=512)
    c = build_cache(wl, n_rows=1500)
    q = wl.attn_query()
    rng = np.random.default_rng(72)
    idx = np.stack([np.sort(rng.choice(1500, 512, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    idx[5, 0, ::2] = -1
    wc, ws, wcr, wsr = window_cache(B, 160, 512, seed=72)
    end = rng.integers(0, 200, size=(B, 1)).astype(np.int32)
    ref_o, ref_l = oracle.sparse_attend(q, c["codes_ref"], c["scales_ref"], idx, wl.softmax_scale,
                                        swa=(wcr, wsr, end, 128))
    out, lse = csa2.sparse_attend(to_dev(q, torch.bfloat16), c["codes"], c["scales"], to_dev(idx), wl.softmax_scale,
                                  out_dtype=torch.float32, swa=csa2.Swa(wc, ws, to_dev(end), 128))
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)
