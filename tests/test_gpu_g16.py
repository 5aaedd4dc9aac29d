"""GPU parity of the pages' FP4 layout: E2M1 codes with one E4M3 scale per 16 channels of
each entry and no global scale ("FP4 Main KV Cache To Halve Storage Again").

Bars as for the per-channel layout: codes, scale bytes and dequantised values bit-exact;
attention on the bf16 MFMA path within 2e-3 max-abs-relative of the fp64 oracle (fp32
output), bf16 output within 2e-3 * max|ref| plus half a bf16 ulp; the fp32 path within
1e-5; layer groups by the near-tie rule on the selections and the attention bar on the
GPU's own selection.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (DEV, check_pool, check_pooled_reindex, check_topk_near_tie, max_abs_rel, to_dev)

pytestmark = pytest.mark.gpu

csa2 = pytest.importorskip("compressed_sparse_attention_csa2_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert csa2.device_check() == 0, "not a gfx950 device"


def g16_cache(x, n_max=None):
    """x [B][T][D] fp32 -> device (codes, gscales) by the library and the oracle's bytes,
    checked equal."""
    B, T, D = x.shape
    n_max = T if n_max is None else n_max
    cr, gr = oracle.quantize_fp4_g16(x, n_max=n_max)
    codes = torch.zeros((B, n_max, D // 2), dtype=torch.uint8, device=DEV)
    gs = torch.zeros((B, n_max, D // 16), dtype=torch.uint8, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_G16, to_dev(x), codes, gs)
    torch.cuda.synchronize()
    assert np.array_equal(gs.cpu().numpy(), gr)
    assert np.array_equal(codes.cpu().numpy(), cr)
    return codes, gs, cr, gr


# ------------------------------------------------------------------------------ codec
@pytest.mark.parametrize("D,n", [(512, 3001), (128, 777), (256, 64)])
def test_quantize_g16_bitexact(D, n):
    wl = workloads.workload("full64k", B=2, D=D)
    x = np.stack([wl.main_kv(b, rows=n) for b in range(2)])
    g16_cache(x)


def test_quantize_g16_special_values_bf16_strided_and_append():
    x = np.zeros((1, 5, 64), np.float32)
    x[0, 0, :16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, -0.1, -0.0, 1e-30, -6.0, 3.0, 0.5, 1e4, -1e4]
    x[0, 0, 16:32] = 6 * 2.0 ** -10                               # scale rounds to 0 -> zero group
    x[0, 0, 32:48] = 6.375                                        # scale rounds down, values saturate
    x[0, 0, 48:64] = np.linspace(-3 * 2.0 ** -9, 3 * 2.0 ** -9, 16)  # subnormal scale
    x[0, 1:] = np.linspace(-300, 300, 4 * 64, dtype=np.float32).reshape(4, 64)
    cr, gr = oracle.quantize_fp4_g16(x, n_max=9)
    big = np.zeros((1, 5, 80), np.float32)                        # row stride 80 > D
    big[:, :, :64] = x
    codes = torch.zeros((1, 9, 32), dtype=torch.uint8, device=DEV)
    gs = torch.zeros((1, 9, 4), dtype=torch.uint8, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_G16, to_dev(big)[:, :, :64], codes, gs)
    # append 4 bf16 rows at n0 = 5
    rng = np.random.default_rng(1)
    new = torch.from_numpy(rng.normal(size=(1, 4, 64)).astype(np.float32) * 3).to(torch.bfloat16)
    oracle.quantize_fp4_g16(new.float().numpy(), n_max=9, n0=np.array([5], np.int32), codes=cr, gscales=gr)
    csa2.quantize_kv(csa2.FMT_FP4_G16, new.to(DEV), codes, gs, n0=to_dev(np.array([5], np.int32)))
    torch.cuda.synchronize()
    assert np.array_equal(gs.cpu().numpy(), gr)
    assert np.array_equal(codes.cpu().numpy(), cr)


def test_gather_dequant_g16_bitexact():
    wl = workloads.workload("full64k", B=2)
    x = np.stack([wl.main_kv(b, rows=900) for b in range(2)])
    codes, gs, cr, gr = g16_cache(x)
    rng = np.random.default_rng(5)
    idx = rng.integers(-1, 900, size=(2, 3, 40)).astype(np.int32)
    idx[0, 0, 0] = 950                                            # out of range -> 0
    ref = oracle.gather_dequant(cr, gr, idx)
    got = csa2.gather_dequant(codes, gs, to_dev(idx)).cpu().numpy()
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------------------ attention
@pytest.mark.parametrize("K,D", [(512, 512), (100, 512), (1024, 512), (37, 512), (2048, 512), (600, 256),
                                 (512, 128)])
def test_sparse_attend_g16_bf16(K, D):
    wl = workloads.workload("full64k", B=2, K=K, D=D)
    x = np.stack([wl.main_kv(b, rows=3000) for b in range(2)])
    codes, gs, cr, gr = g16_cache(x)
    q = wl.attn_query()
    rng = np.random.default_rng(K + D)
    idx = np.stack([np.sort(rng.choice(3000, K, replace=False)) for _ in range(2)]).astype(np.int32)[:, None]
    idx[1, 0, ::5] = -1
    ref_o, ref_l = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale)
    qd = to_dev(q, torch.bfloat16)
    out, lse = csa2.sparse_attend(qd, codes, gs, to_dev(idx), wl.softmax_scale, out_dtype=torch.float32)
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)
    ob, _ = csa2.sparse_attend(qd, codes, gs, to_dev(idx), wl.softmax_scale, out_dtype=torch.bfloat16)
    ob = ob.float().cpu().numpy()
    assert np.all(np.abs(ob - ref_o) <= 2e-3 * np.abs(ref_o).max() + np.abs(ref_o) * 2.0 ** -8)


def test_sparse_attend_g16_many_rows():
    """72 rows: more attention blocks than fit one round on the chip, where the G16 layout runs
    the undivided grid (the decode shapes above take the channel split)."""
    B = 72
    wl = workloads.workload("full64k", B=B, K=512)
    x = np.stack([wl.main_kv(b, rows=900) for b in range(B)])
    codes, gs, cr, gr = g16_cache(x)
    q = wl.attn_query()
    rng = np.random.default_rng(1672)
    idx = np.stack([np.sort(rng.choice(900, 512, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    idx[7, 0, ::4] = -1
    ref_o, ref_l = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale)
    out, lse = csa2.sparse_attend(to_dev(q, torch.bfloat16), codes, gs, to_dev(idx), wl.softmax_scale,
                                  out_dtype=torch.float32)
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)


def test_sparse_attend_g16_subnormal_scales():
    """Small entries whose group scales are subnormal E4M3 codes (m * 2^-9): the output is
    built from them alone, so a wrong subnormal decode shows at full relative size."""
    wl = workloads.workload("full64k", B=1, K=512)
    x = (wl.main_kv(0, rows=2000) * 0.015)[None].astype(np.float32)
    codes, gs, cr, gr = g16_cache(x)
    assert np.mean(gr < 8) > 0.9                                  # mostly subnormal scale codes
    q = wl.attn_query()
    rng = np.random.default_rng(9)
    idx = np.sort(rng.choice(2000, 512, replace=False)).astype(np.int32)[None, None]
    ref_o, ref_l = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale)
    out, lse = csa2.sparse_attend(to_dev(q, torch.bfloat16), codes, gs, to_dev(idx), wl.softmax_scale,
                                  out_dtype=torch.float32)
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 2e-3
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=2e-3, atol=2e-3)


def test_sparse_attend_g16_skipped_rows_read_no_scale():
    """Skipped entries never contribute, even when the cache rows they would stand in for
    hold NaN scale bytes (E4M3 0x7F)."""
    wl = workloads.workload("full64k", B=1, K=512)
    x = wl.main_kv(0, rows=700)[None]
    codes, gs, cr, gr = g16_cache(x)
    gs[0, 0] = 0x7F                                               # row 0: NaN scales
    gr = gr.copy()
    gr[0, 0] = 0x7F
    q = wl.attn_query()
    idx = np.full((1, 1, 512), -1, np.int32)
    idx[0, 0, :300] = np.arange(1, 301)
    ref_o, _ = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale)
    out, _ = csa2.sparse_attend(to_dev(q, torch.bfloat16), codes, gs, to_dev(idx), wl.softmax_scale,
                                out_dtype=torch.float32)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o)) and max_abs_rel(o, ref_o) <= 2e-3
    empty = torch.full((1, 1, 512), -1, dtype=torch.int32, device=DEV)
    out, lse = csa2.sparse_attend(to_dev(q, torch.bfloat16), codes, gs, empty, wl.softmax_scale,
                                  out_dtype=torch.float32)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_sparse_attend_g16_fp32():
    wl = workloads.WORKLOADS["tiny"]
    x = wl.main_kv(0)[None]
    codes, gs, cr, gr = g16_cache(x)
    q = wl.attn_query()
    rng = np.random.default_rng(2)
    idx = np.sort(rng.choice(wl.N, 64, replace=False)).astype(np.int32)[None, None]
    idx[0, 0, -3:] = -1
    ref_o, ref_l = oracle.sparse_attend(q, cr, gr, idx, wl.softmax_scale)
    out, lse = csa2.sparse_attend(to_dev(q), codes, gs, to_dev(idx), wl.softmax_scale)
    assert max_abs_rel(out.cpu().numpy(), ref_o) <= 1e-5
    assert np.allclose(lse.cpu().numpy(), ref_l, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------------------ layer group
@pytest.mark.parametrize("pool", [None, (8, 128)])
def test_layer_group_g16(pool):
    wl = workloads.workload("group128k", B=3, N=20000, K=256)
    x = np.stack([wl.main_kv(b, rows=wl.N) for b in range(3)])
    kf = np.stack([wl.index_keys(b, rows=wl.N) for b in range(3)])
    codes, gs, cr, gr = g16_cache(x)
    k8r, ksr = oracle.quantize_fp8(kf)
    k8 = torch.empty((3, wl.N, 64), dtype=torch.uint8, device=DEV)
    ks = torch.empty((3, wl.N), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, to_dev(kf), k8, ks)
    nk = np.array([20000, 15001, 900], np.int32)
    modes = ["full", "reindex", "reuse", "reindex"]
    layers, ref_layers = [], []
    for i, m in enumerate(modes):
        qi, w, qa = wl.index_query(i), wl.head_weights(i), wl.attn_query(i)
        ref_layers.append(dict(mode=m, q_idx=qi, w=w, q_attn=qa))
        L = dict(mode=m, q_idx=to_dev(qi, torch.bfloat16), w=to_dev(w), q_attn=to_dev(qa, torch.bfloat16))
        if m == "full" and pool:
            L["pool"] = torch.full((3, pool[0] * pool[1]), -7, dtype=torch.int32, device=DEV)
        layers.append(L)
    cache = csa2.GroupCache(to_dev(nk), codes, gs, k8, ks, wl.K, wl.softmax_scale, pool=pool)
    csa2.layer_group(layers, cache, out_dtype=torch.float32)
    torch.cuda.synchronize()
    gpool = g_idx = None
    for i, (L, RL) in enumerate(zip(layers, ref_layers)):
        if L["mode"] == "full" or (L["mode"] == "reindex" and not pool):
            s = oracle.index_score(oracle.PREC_FP8, RL["q_idx"], RL["w"], k8r, ksr, nk)
            g_idx = L["idx"].cpu().numpy()
            check_topk_near_tie(g_idx, s, wl.K)
            if pool and L["mode"] == "full":
                gpool = L["pool"].cpu().numpy()
                check_pool(gpool, s, pool[0], pool[1], nk)
        elif L["mode"] == "reindex":
            g_idx = L["idx"].cpu().numpy()
            check_pooled_reindex(g_idx, RL["q_idx"], RL["w"], k8r, ksr, nk, gpool, wl.K)
        ro, _ = oracle.sparse_attend(RL["q_attn"], cr, gr, g_idx, wl.softmax_scale)
        assert max_abs_rel(L["out"].cpu().numpy(), ro) <= 2e-3, i
