"""CSA2 CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this package.  The product path (``compressed_sparse_attention_csa2_amd``) never
does: it shares no code, header, table or helper with it.

The arithmetic lives in ``csa2_oracle.c`` (plain C, fp64, built with gcc
``-O2 -fopenmp -ffp-contract=off``); this module only marshals numpy arrays and composes
the per-step functions into the layer modes and the two-level indexer, following
"Detailed Notes On DeepSeek V4 Point 1 Flash In Simple Words" ("The Three Modes Full
Reindex And Reuse", "Hierarchical Sparse Indexer In Simple Terms") and
"DeepSeek-V4.1-Flash 技术解读" 3.3 (mode table and the caption saying which layer each mode
borrows from).

Pins: tests/test_oracle_*.py check every function here against closed forms, exhaustive
tables, brute force and library special cases (dense attention, torch's E4M3 cast).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_lib = None

PREC_FP32, PREC_FP8, PREC_FP4 = 0, 1, 2
FMT_FP4_PER_CHANNEL, FMT_FP4_G16 = 0, 2


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        i, i64, f, d, p = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
        L.orc_e2m1_value.argtypes, L.orc_e2m1_value.restype = [i], d
        L.orc_e2m1_encode.argtypes, L.orc_e2m1_encode.restype = [f], i
        L.orc_e4m3_value.argtypes, L.orc_e4m3_value.restype = [i], d
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [f], i
        L.orc_quantize_fp4.argtypes = [i, i, i, p, i64, i64, p, i64, p, p, i]
        L.orc_quantize_fp8.argtypes = [i, i, i, p, i64, i64, p, i64, p, p]
        L.orc_quantize_fp4_rows.argtypes = [i, i, i, p, i64, i64, p, i64, p, p]
        L.orc_quantize_index_query.argtypes = [i, i, p, p, p]
        L.orc_quantize_fp4_g16.argtypes = [i, i, i, p, i64, i64, p, i64, p, p]
        L.orc_gather_dequant.argtypes = [i, i, i, i, i, p, p, i64, p, p]
        L.orc_index_score.argtypes = [i, i, i, i, i, p, p, p, p, i64, p, p, p, i, p]
        L.orc_topk.argtypes = [i, i, i64, p, p, i, p, p]
        L.orc_sparse_attend.argtypes = [i, i, i, i, i, p, p, p, i64, p, i, p, p, i64, p, i, d, p, p]
        L.orc_coarse_keys.argtypes = [i, i64, p, i, i, p, p, p, p]
        L.orc_num_threads.argtypes, L.orc_num_threads.restype = [], i
        for fn in ("orc_quantize_fp4", "orc_quantize_fp4_g16", "orc_quantize_fp8", "orc_quantize_fp4_rows",
                   "orc_quantize_index_query",
                   "orc_gather_dequant", "orc_index_score", "orc_topk", "orc_sparse_attend", "orc_coarse_keys"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return _load().orc_num_threads()


# ---------------------------------------------------------------------------- codecs
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e2m1_encode(y: float) -> int:
    return _load().orc_e2m1_encode(float(y))


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e4m3_encode(y: float) -> int:
    return _load().orc_e4m3_encode(float(y))


# ---------------------------------------------------------------------------- write side
def quantize_fp4(x, n_max=None, n0=None, scales=None, codes=None):
    """x [B][T][D] -> (codes [B][n_max][D/2] u8, scales [B][D] f32).

    scales None: computed from x (absmax/6 per channel); else used as given (append)."""
    x = _c(x, np.float32)
    B, T, D = x.shape
    n_max = T if n_max is None else n_max
    compute = scales is None
    scales = np.zeros((B, D), np.float32) if compute else _c(scales, np.float32).copy()
    codes = np.zeros((B, n_max, D // 2), np.uint8) if codes is None else codes
    assert codes.shape == (B, n_max, D // 2) and codes.flags["C_CONTIGUOUS"]
    n0a = None if n0 is None else _c(n0, np.int32)
    _load().orc_quantize_fp4(B, T, D, _p(x), T * D, D, _p(n0a), n_max, _p(codes), _p(scales), int(compute))
    return codes, scales


def quantize_fp4_g16(x, n_max=None, n0=None, codes=None, gscales=None):
    """x [B][T][D] -> (codes [B][n_max][D/2] u8, gscales [B][n_max][D/16] u8): the pages'
    layout, one E4M3 scale per 16 channels of each entry (see orc_quantize_fp4_g16)."""
    x = _c(x, np.float32)
    B, T, D = x.shape
    assert D % 16 == 0
    n_max = T if n_max is None else n_max
    codes = np.zeros((B, n_max, D // 2), np.uint8) if codes is None else codes
    gscales = np.zeros((B, n_max, D // 16), np.uint8) if gscales is None else gscales
    assert codes.flags["C_CONTIGUOUS"] and gscales.flags["C_CONTIGUOUS"]
    n0a = None if n0 is None else _c(n0, np.int32)
    _load().orc_quantize_fp4_g16(B, T, D, _p(x), T * D, D, _p(n0a), n_max, _p(codes), _p(gscales))
    return codes, gscales


def _kv_scales(scales):
    """(format, contiguous scales): uint8 scales are the per-16-channel E4M3 layout
    [B][n_max][D/16], anything else the per-channel fp32 scales [B][D]."""
    a = np.asarray(scales)
    if a.dtype == np.uint8:
        return FMT_FP4_G16, _c(a, np.uint8)
    return FMT_FP4_PER_CHANNEL, _c(a, np.float32)


def quantize_fp4_rows(x, n_max=None, n0=None, codes=None, scales=None):
    """x [B][T][D] -> (codes [B][n_max][D/2] u8, scales [B][n_max] f32): E2M1 with one
    absmax/6 scale per row (the 4-bit indexer keys, orc_quantize_fp4_rows)."""
    x = _c(x, np.float32)
    B, T, D = x.shape
    assert D % 2 == 0
    n_max = T if n_max is None else n_max
    codes = np.zeros((B, n_max, D // 2), np.uint8) if codes is None else codes
    scales = np.zeros((B, n_max), np.float32) if scales is None else scales
    assert codes.flags["C_CONTIGUOUS"] and scales.flags["C_CONTIGUOUS"]
    n0a = None if n0 is None else _c(n0, np.int32)
    _load().orc_quantize_fp4_rows(B, T, D, _p(x), T * D, D, _p(n0a), n_max, _p(codes), _p(scales))
    return codes, scales


def quantize_fp8(x, n_max=None, n0=None, codes=None, scales=None):
    """x [B][T][D] -> (codes [B][n_max][D] u8, scales [B][n_max] f32); per-row absmax/448."""
    x = _c(x, np.float32)
    B, T, D = x.shape
    n_max = T if n_max is None else n_max
    codes = np.zeros((B, n_max, D), np.uint8) if codes is None else codes
    scales = np.zeros((B, n_max), np.float32) if scales is None else scales
    assert codes.flags["C_CONTIGUOUS"] and scales.flags["C_CONTIGUOUS"]
    n0a = None if n0 is None else _c(n0, np.int32)
    _load().orc_quantize_fp8(B, T, D, _p(x), T * D, D, _p(n0a), n_max, _p(codes), _p(scales))
    return codes, scales


def quantize_index_query(q):
    """q [..][dk] -> (q8 codes, sq scales): E4M3 per row with absmax/448."""
    q = _c(q, np.float32)
    dk = q.shape[-1]
    rows = q.size // dk
    q8 = np.zeros(q.shape, np.uint8)
    sq = np.zeros(q.shape[:-1], np.float32)
    _load().orc_quantize_index_query(rows, dk, _p(q), _p(q8), _p(sq))
    return q8, sq


def gather_dequant(codes, scales, idx):
    fmt, scales = _kv_scales(scales)
    codes, idx = _c(codes, np.uint8), _c(idx, np.int32)
    B, n_max, Dh = codes.shape
    _, T, K = idx.shape
    out = np.zeros((B, T, K, 2 * Dh), np.float32)
    _load().orc_gather_dequant(fmt, B, T, K, 2 * Dh, _p(codes), _p(scales), n_max, _p(idx), _p(out))
    return out


# ---------------------------------------------------------------------------- indexer
def index_score(prec, q, w, k, k_scale, n_keys, q_limit=None, cand=None):
    """Scores [B][T][ncols] float64 (-inf where not visible).

    prec PREC_FP32: k is [B][n_max][dk] f32; PREC_FP8: k is E4M3 codes + k_scale [B][n_max];
    PREC_FP4: k is packed E2M1 codes [B][n_max][dk/2] + k_scale [B][n_max]."""
    q = _c(q, np.float32)
    B, T, H, dk = q.shape
    w = _c(w, np.float32)
    k = _c(k, np.float32 if prec == PREC_FP32 else np.uint8)
    n_max = k.shape[1]
    ks = None if k_scale is None else _c(k_scale, np.float32)
    nk = _c(n_keys, np.int32)
    ql = None if q_limit is None else _c(q_limit, np.int32)
    ca = None if cand is None else _c(cand, np.int32)
    C = 0 if ca is None else ca.shape[-1]
    ncols = C if ca is not None else n_max
    out = np.empty((B, T, ncols), np.float64)
    _load().orc_index_score(prec, B, T, H, dk, _p(q), _p(w), _p(k), _p(ks), n_max, _p(nk), _p(ql), _p(ca), C,
                            _p(out))
    return out


def topk(scores, K, cand=None, want_values=False):
    s = _c(scores, np.float64)
    B, T, ncols = s.shape
    ca = None if cand is None else _c(cand, np.int32)
    idx = np.empty((B, T, K), np.int32)
    val = np.empty((B, T, K), np.float64) if want_values else None
    _load().orc_topk(B, T, ncols, _p(s), _p(ca), K, _p(idx), _p(val))
    return (idx, val) if want_values else idx


# ---------------------------------------------------------------------------- attention
def sparse_attend(q, codes, scales, idx, softmax_scale, swa=None):
    """(out [B][T][Hq][D] float64, lse [B][T][Hq] float64).  scales: fp32 [B][D] (one per
    channel) or uint8 [B][n_max][D/16] (E4M3 per 16 channels of each entry).
    swa: None, or (swa_codes [B][n][D] u8, swa_scales [B][n] f32, swa_end [B][T] i32,
    window): the layer's sliding-window entries, attended in the same softmax."""
    q = _c(q, np.float32)
    B, T, Hq, D = q.shape
    fmt, scales = _kv_scales(scales)
    codes, idx = _c(codes, np.uint8), _c(idx, np.int32)
    n_max = codes.shape[1]
    K = idx.shape[-1]
    out = np.empty((B, T, Hq, D), np.float64)
    lse = np.empty((B, T, Hq), np.float64)
    sc = ss = se = None
    sn, win = 0, 0
    if swa is not None:
        sc, ss, se, win = _c(swa[0], np.uint8), _c(swa[1], np.float32), _c(swa[2], np.int32), int(swa[3])
        assert sc.shape[0] == B and sc.shape[2] == D and se.shape == (B, T)
        sn = sc.shape[1]
    _load().orc_sparse_attend(fmt, B, T, Hq, D, _p(q), _p(codes), _p(scales), n_max, _p(idx), K, _p(sc), _p(ss),
                              sn, _p(se), win, float(softmax_scale), _p(out), _p(lse))
    return out, lse


# ---------------------------------------------------------------------------- modes
FULL, REINDEX, REUSE = "full", "reindex", "reuse"


def check_schedule(modes):
    """The mode-order rule: the first layer is Full; a Reindex layer needs an earlier Full
    layer (whose main KV and indexer keys it shares); a Reuse layer needs an earlier
    indexing layer (Full or Reindex) whose Top-K it takes unchanged."""
    seen_full = seen_index = False
    for m in modes:
        if m == FULL:
            seen_full = seen_index = True
        elif m == REINDEX:
            if not seen_full:
                return False
            seen_index = True
        elif m == REUSE:
            if not seen_index:
                return False
        else:
            return False
    return len(modes) > 0


def block_max(scores, block):
    """[B][T][n] scores -> [B][T][ceil(n / block)]: the largest score in each block of
    `block` consecutive positions, -inf where the block holds no visible score.
    "Hierarchical Sparse Indexer In Simple Terms": a block is represented by its best
    entry's score."""
    s = np.asarray(scores, np.float64)
    B, T, n = s.shape
    nb = (n + block - 1) // block
    pad = np.full((B, T, nb * block), -np.inf)
    pad[..., :n] = s
    return pad.reshape(B, T, nb, block).max(axis=3)


def pool_positions(scores, block, pool_blocks, n_keys):
    """The candidate pool a Full layer leaves for later Reindex layers: the `pool_blocks`
    blocks with the largest block maxima (lowest block index on ties), expanded to their
    positions in ascending order (-1 past n_keys or for missing blocks).  Same source."""
    blocks = topk(block_max(scores, block), pool_blocks)
    return expand_blocks(blocks, block, n_keys)


def layer_group(layers, cache, prec, K, softmax_scale, pool=None):
    """Run the layers in order over one shared cache.

    layers: list of dicts {mode, q_idx, w, q_attn} and optionally swa (the layer's own
    sliding-window cache, as for sparse_attend); cache: dict {k, k_scale, n_keys, codes,
    scales}.  Full and Reindex score the shared indexer keys with their own query and
    take a fresh Top-K; Reuse takes the most recent indexing layer's Top-K unchanged.
    Every mode then attends over the shared main KV with its own attention query.
    pool = (block, pool_blocks): every Full layer also leaves the pool of its best blocks
    (pool_positions) and the Reindex layers after it score only the pool's positions.
    T query tokens per sequence (the second dim of q_attn; T > 1 for draft verification, as
    DSpark's five parallel drafts need in "Detailed Notes", DSpark section): their own
    entries are the cache's last T, so token t sees positions < n_keys - (T - 1 - t).
    Returns a list of dicts {idx, out, lse} (plus 'pool' for Full layers with a pool)."""
    modes = [L["mode"] for L in layers]
    if not check_schedule(modes):
        raise ValueError("invalid mode schedule %r" % (modes,))
    nk = _c(cache["n_keys"], np.int32)
    T = np.asarray(layers[0]["q_attn"]).shape[1]
    q_limit = None
    if T > 1:
        q_limit = (nk[:, None] - T + np.arange(T, dtype=np.int32)[None, :]).astype(np.int32)
    results, last_idx, cand = [], None, None
    for L in layers:
        res = {}
        if L["mode"] == FULL or (L["mode"] == REINDEX and cand is None):
            s = index_score(prec, L["q_idx"], L["w"], cache["k"], cache["k_scale"], nk, q_limit=q_limit)
            last_idx = topk(s, K)
            if L["mode"] == FULL and pool is not None:
                # a row's pool holds only positions it can see
                cand = pool_positions(s, pool[0], pool[1], nk if q_limit is None else q_limit + 1)
                res["pool"] = cand
        elif L["mode"] == REINDEX:
            s = index_score(prec, L["q_idx"], L["w"], cache["k"], cache["k_scale"], nk, q_limit=q_limit, cand=cand)
            last_idx = topk(s, K, cand=cand)
        out, lse = sparse_attend(L["q_attn"], cache["codes"], cache["scales"], last_idx, softmax_scale,
                                 swa=L.get("swa"))
        res.update({"idx": last_idx, "out": out, "lse": lse})
        results.append(res)
    return results


# ---------------------------------------------------------------------------- two-level indexer
def coarse_keys(k8, k_scale, n_keys, block):
    k8, ks, nk = _c(k8, np.uint8), _c(k_scale, np.float32), _c(n_keys, np.int32)
    B, n_max, dk = k8.shape
    nb = (n_max + block - 1) // block
    kb8 = np.zeros((B, nb, dk), np.uint8)
    kbs = np.zeros((B, nb), np.float32)
    _load().orc_coarse_keys(B, n_max, _p(nk), dk, block, _p(k8), _p(ks), _p(kb8), _p(kbs))
    return kb8, kbs


def expand_blocks(block_idx, block, n_keys):
    """Candidate positions of the selected blocks: block ascending, then position
    ascending; positions at or past n_keys ([B], or [B][T] per query row) and padded
    blocks become -1."""
    B, T, KB = block_idx.shape
    cand = np.full((B, T, KB * block), -1, np.int32)
    off = np.arange(block, dtype=np.int64)
    nk = np.asarray(n_keys)
    for b in range(B):
        for t in range(T):
            lim = nk[b, t] if nk.ndim == 2 else nk[b]
            for i, blk in enumerate(block_idx[b, t]):
                if blk < 0:
                    continue
                pos = blk * block + off
                pos[pos >= lim] = -1
                cand[b, t, i * block:(i + 1) * block] = pos
    return cand


def hier_select(q, w, k8, k_scale, kb8, kb_scale, n_keys, block, block_topk, K):
    """Two-level Top-K: score the coarse keys, keep the best `block_topk` blocks (lowest
    block index on ties), score every position inside them exactly and keep the best K
    (lowest position on ties).  Returns (idx [B][T][K], block_idx [B][T][block_topk])."""
    n_keys = _c(n_keys, np.int32)
    nb_keys = (n_keys + block - 1) // block
    cs = index_score(PREC_FP8, q, w, kb8, kb_scale, nb_keys)
    blk = topk(cs, block_topk)
    cand = expand_blocks(blk, block, n_keys)
    fs = index_score(PREC_FP8, q, w, k8, k_scale, n_keys, cand=cand)
    return topk(fs, K, cand=cand), blk
