"""Shared helpers of the GPU parity tests: seeded inputs on both sides and the acceptance
rules (bit-exact bytes, near-tie Top-K acceptance, max-abs-relative attention error)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

DEV = "cuda"


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def fp8_score_bound(q, w, k8, ks, n_keys=None):
    """Per-element error scale of an fp32 evaluation of the fp8 score:
    sk_j * sum_h |w_h sq_h| sum_d |q8_hd| |k8_jd|  ([B][T][n])."""
    q8, sq = oracle.quantize_index_query(q)
    qd = np.abs(e4m3_to_f64(q8)) * (np.abs(w.astype(np.float64)) * sq.astype(np.float64))[..., None]
    kd = np.abs(e4m3_to_f64(k8))
    qs = qd.sum(axis=2)  # sum over heads of |c_h| |q8_h|  -> [B][T][dk]
    return np.einsum("btd,bjd->btj", qs, kd) * ks.astype(np.float64)[:, None, :]


def e2m1_unpack_f64(codes):
    """Packed E2M1 codes [..][n/2] -> values [..][n] (lower index in the low nibble)."""
    tab = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1).astype(np.int64)
    return np.where(c & 8, -1.0, 1.0) * tab[c & 7]


def fp4_score_bound(q, w, k4, ks):
    """As fp8_score_bound for the 4-bit indexer: sk_j * sum_h |w_h sq_h| sum_d |q4_hd| |k4_jd|,
    the query quantised per (token, head) to E2M1 with absmax/6 ([B][T][n])."""
    B, T, H, dk = q.shape
    qc, sq = oracle.quantize_fp4_rows(np.ascontiguousarray(q, np.float32).reshape(1, B * T * H, dk))
    q4 = np.abs(e2m1_unpack_f64(qc)).reshape(B, T, H, dk)
    qd = q4 * (np.abs(w.astype(np.float64)) * sq.reshape(B, T, H).astype(np.float64))[..., None]
    kd = np.abs(e2m1_unpack_f64(k4))
    return np.einsum("btd,bjd->btj", qd.sum(axis=2), kd) * ks.astype(np.float64)[:, None, :]


def check_topk_near_tie(gpu_idx, ref_scores, K, rel=1e-3, n_vis=None):
    """Near-tie acceptance rule: with tau the reference K-th score and delta = rel*|tau|, the GPU set G
    must have min(K, n_vis) members, contain every j with s_j > tau + delta and lie inside
    {j : s_j >= tau - delta}.  Also: ascending order, -1 padding."""
    B, T, _ = gpu_idx.shape
    exact_rows = 0
    for b in range(B):
        for t in range(T):
            s = ref_scores[b, t]
            vis = np.isfinite(s) | (s == np.inf)
            nv = int(vis.sum())
            g = gpu_idx[b, t]
            keep = min(K, nv)
            assert np.all(g[keep:] == -1), (b, t)
            sel = g[:keep]
            assert np.all(sel >= 0) and np.all(np.diff(sel) > 0), (b, t)
            if keep == 0:
                continue
            order = np.lexsort((np.arange(len(s)), -np.where(vis, s, -np.inf)))
            tau = s[order[keep - 1]]
            delta = rel * abs(tau)
            must = np.nonzero(vis & (s > tau + delta))[0]
            may = vis & (s >= tau - delta)
            assert np.all(np.isin(must, sel)), (b, t, "missing a clear winner")
            assert np.all(may[sel]), (b, t, "selected a clear loser")
            ref_set = np.sort(order[:keep])
            exact_rows += int(np.array_equal(ref_set, sel))
    return exact_rows


def max_abs_rel(out, ref):
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(np.asarray(out, np.float64) - ref)) / (den if den > 0 else 1.0))


def build_cache(wl, n_rows=None, seqs=None):
    """Main-KV and indexer-key caches of a workload on both sides from the same drawn
    values: returns dict with the fp32 inputs, the oracle's bytes and device tensors
    quantised by the library."""
    import compressed_sparse_attention_csa2_amd as csa2
    n = wl.N if n_rows is None else n_rows
    seqs = list(range(wl.B)) if seqs is None else seqs
    B = len(seqs)
    x = np.stack([wl.main_kv(b, rows=n) for b in seqs])
    kf = np.stack([wl.index_keys(b, rows=n) for b in seqs])
    res = {"x": x, "kf": kf, "n": n}
    res["codes_ref"], res["scales_ref"] = oracle.quantize_fp4(x)
    if wl.index_fp8:
        res["k8_ref"], res["ks_ref"] = oracle.quantize_fp8(kf)
    xd = to_dev(x)
    codes = torch.empty((B, n, wl.D // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((B, wl.D), dtype=torch.float32, device=DEV)
    csa2.quantize_kv(csa2.FMT_FP4_PER_CHANNEL, xd, codes, scales)
    del xd
    res["codes"], res["scales"] = codes, scales
    kd = to_dev(kf)
    if wl.index_fp8:
        k8 = torch.empty((B, n, wl.dk), dtype=torch.uint8, device=DEV)
        ks = torch.empty((B, n), dtype=torch.float32, device=DEV)
        csa2.quantize_kv(csa2.FMT_FP8_PER_TOKEN, kd, k8, ks)
        res["k8"], res["ks"] = k8, ks
    else:
        res["kdev"] = kd
    return res


def check_pool(gpool, s_ref, block, blocks, nk):
    """A candidate pool gpool [B][blocks*block] from the GPU against the oracle's Full scores
    s_ref [B][1][n]: its block list by the near-tie rule on the block maxima, its positions
    exactly the expansion of that list."""
    bm = oracle.block_max(s_ref, block)
    for b in range(gpool.shape[0]):
        p = gpool[b]
        first = p[::block]
        blk = np.where(first >= 0, first // block, -1).astype(np.int32)
        assert np.array_equal(oracle.expand_blocks(blk[None, None], block, nk[b:b + 1])[0, 0], p), b
        check_topk_near_tie(blk[None, None], bm[b:b + 1], blocks)


def check_pooled_reindex(g_idx, q, w, k8, ks, nk, gpool, K):
    """A Reindex selection against the oracle's scores of the GPU's pool positions (near-tie
    rule on the pool), and inside the pool."""
    n = k8.shape[1]
    fs = oracle.index_score(oracle.PREC_FP8, q, w, k8, ks, nk, cand=gpool[:, None])
    full = np.full((len(nk), 1, n), -np.inf)
    for b in range(len(nk)):
        ok = gpool[b] >= 0
        full[b, 0, gpool[b][ok]] = fs[b, 0][ok]
    check_topk_near_tie(g_idx, full, K)
    for b in range(len(nk)):
        sel = g_idx[b, 0]
        assert np.all(np.isin(sel[sel >= 0], gpool[b])), b


def single_head_edge_queries(q):
    """Index queries [B][T][32][64] where row r = (b, t) keeps only head r % 32, bf16-exact,
    scaled by kind r % 4: 1e-27 (a per-head scale below 2^-92), spread over six decades
    (many E4M3 subnormal codes), 1e30, or as drawn.  Every other head is zero."""
    rng = np.random.default_rng(21)
    B, T, H, dk = q.shape
    out = np.zeros((B, T, H, dk), np.float32)
    for r in range(B * T):
        b, t, h = r // T, r % T, r % H
        v = q[b, t, h].astype(np.float32)
        kind = r % 4
        if kind == 0:
            v = v * np.float32(1e-27)
        elif kind == 1:
            v = v * (10.0 ** rng.uniform(-6, 0, size=dk)).astype(np.float32)
        elif kind == 2:
            v = v * np.float32(1e30)
        out[b, t, h] = v
    return torch.from_numpy(out).to(torch.bfloat16).float().numpy()


def one_hot_keys(B, n, dk=64):
    """Keys [B][n][dk] with key j = unit vector along dim j % dk: each score of a one-head
    query is then a single product, exact up to the rounding of the final scaling."""
    k = np.zeros((B, n, dk), np.float32)
    j = np.arange(n)
    k[:, j, j % dk] = 1.0
    return k
