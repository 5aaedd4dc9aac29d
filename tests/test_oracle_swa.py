"""Pins of the oracle's sliding-window part of the attention: every layer also attends to
its own most recent entries ("CSA2 In Simple Terms"; window 128 in "Model Setup Numbers";
the window cache stays 8-bit in "FP4 Main KV Cache"), in the same softmax as the selected
entries.

Entries are built exactly representable in their formats, so the dequantised rows equal
the inputs and every result can be checked against dense fp64 softmax attention (torch)
over the rows that should be attended: the window bounds, the clamping at the start of a
sequence and at the cache end, the union with the selected entries, the merge identity,
and the empty cases."""
import numpy as np
import torch

import oracle

E4M3_GRID = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 3.0, 3.5, 4.0, 6.0, 8.0, 12.0], np.float32)


def _exact_fp8_rows(rng, B, n, D):
    """Rows on the E4M3 grid with an exact power-of-two per-row scale (absmax 448 * 2^k)."""
    v = E4M3_GRID[rng.integers(0, len(E4M3_GRID), size=(B, n, D))] * rng.choice([-1.0, 1.0], size=(B, n, D))
    v[:, :, 0] = 448.0                                    # per-row absmax 448: the scale is 2^k exactly
    k = rng.integers(-12, -4, size=(B, n, 1)).astype(np.float32)
    return (v * np.float32(2.0) ** k).astype(np.float32)


def _exact_fp4_rows(rng, B, n, D):
    """Rows on the E2M1 grid times per-channel power-of-two scales (absmax 6 per channel)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    v = grid[rng.integers(0, 8, size=(B, n, D))] * rng.choice([-1.0, 1.0], size=(B, n, D))
    v[:, 0, :] = 6.0
    s = np.float32(2.0) ** rng.integers(-6, -2, size=(B, 1, D)).astype(np.float32)
    return (v * s).astype(np.float32)


def _dense(q, rows, scale):
    kv = torch.from_numpy(np.asarray(rows, np.float64))
    lg = scale * torch.from_numpy(q.astype(np.float64)) @ kv.T
    return (torch.softmax(lg, -1) @ kv).numpy(), torch.logsumexp(lg, -1).numpy()


def _setup(seed=0, B=2, T=1, Hq=4, D=64, n_main=50, n_swa=40):
    rng = np.random.default_rng(seed)
    x = _exact_fp4_rows(rng, B, n_main, D)
    codes, scales = oracle.quantize_fp4(x)
    w = _exact_fp8_rows(rng, B, n_swa, D)
    wc, ws = oracle.quantize_fp8(w)
    q = rng.normal(size=(B, T, Hq, D)).astype(np.float32)
    return rng, x, codes, scales, w, wc, ws, q


def test_rows_are_exact_in_both_formats():
    rng, x, codes, scales, w, wc, ws, q = _setup()
    assert np.array_equal(oracle.gather_dequant(codes, scales, np.arange(50, dtype=np.int32)[None, None]
                                                .repeat(2, 0))[:, 0], x)
    assert np.array_equal(np.vectorize(oracle.e4m3_value)(wc.astype(np.int64)) * ws[..., None], w)


def test_window_only_is_dense_attention_over_the_window_rows():
    rng, x, codes, scales, w, wc, ws, q = _setup()
    idx = np.full((2, 1, 16), -1, np.int32)
    end = np.array([[40], [23]], np.int32)
    out, lse = oracle.sparse_attend(q, codes, scales, idx, 0.1, swa=(wc, ws, end, 16))
    for b, (lo, hi) in enumerate([(24, 40), (7, 23)]):
        ro, rl = _dense(q[b, 0], w[b, lo:hi], 0.1)
        assert np.allclose(out[b, 0], ro, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[b, 0], rl, rtol=1e-12, atol=1e-12)


def test_window_clamps_at_the_sequence_start_and_the_cache_end():
    rng, x, codes, scales, w, wc, ws, q = _setup()
    idx = np.full((2, 1, 4), -1, np.int32)
    end = np.array([[5], [99]], np.int32)                 # 5 < window; 99 > the 40 cached rows
    out, _ = oracle.sparse_attend(q, codes, scales, idx, 0.1, swa=(wc, ws, end, 16))
    assert np.allclose(out[0, 0], _dense(q[0, 0], w[0, 0:5], 0.1)[0], rtol=1e-12, atol=1e-12)
    assert np.allclose(out[1, 0], _dense(q[1, 0], w[1, 24:40], 0.1)[0], rtol=1e-12, atol=1e-12)


def test_union_of_selected_and_window_rows_is_one_softmax():
    rng, x, codes, scales, w, wc, ws, q = _setup(seed=3, T=2)
    idx = np.stack([np.stack([np.sort(rng.choice(50, 12, replace=False)) for _ in range(2)]) for _ in range(2)])
    idx = idx.astype(np.int32)
    idx[1, 0, 3] = -1
    end = np.array([[30, 31], [40, 12]], np.int32)
    out, lse = oracle.sparse_attend(q, codes, scales, idx, 0.07, swa=(wc, ws, end, 8))
    for b in range(2):
        for t in range(2):
            sel = idx[b, t][idx[b, t] >= 0]
            e = end[b, t]
            rows = np.concatenate([x[b, sel], w[b, max(0, e - 8):e]])
            ro, rl = _dense(q[b, t], rows, 0.07)
            assert np.allclose(out[b, t], ro, rtol=1e-12, atol=1e-12)
            assert np.allclose(lse[b, t], rl, rtol=1e-12, atol=1e-12)


def test_merge_identity_and_empty_cases():
    rng, x, codes, scales, w, wc, ws, q = _setup(seed=5)
    idx = np.sort(rng.choice(50, 20, replace=False)).astype(np.int32)[None, None].repeat(2, 0)
    end = np.array([[33], [17]], np.int32)
    o_all, l_all = oracle.sparse_attend(q, codes, scales, idx, 0.1, swa=(wc, ws, end, 16))
    o_s, l_s = oracle.sparse_attend(q, codes, scales, idx, 0.1)
    o_w, l_w = oracle.sparse_attend(q, codes, scales, np.full_like(idx, -1), 0.1, swa=(wc, ws, end, 16))
    m = np.maximum(l_s, l_w)
    a, c = np.exp(l_s - m)[..., None], np.exp(l_w - m)[..., None]
    assert np.allclose(o_all, (a * o_s + c * o_w) / (a + c), rtol=1e-12, atol=1e-12)
    assert np.allclose(l_all, m + np.log(a + c)[..., 0], rtol=1e-12, atol=1e-12)
    # an empty window changes nothing; nothing at all gives 0 and -inf
    o_e, l_e = oracle.sparse_attend(q, codes, scales, idx, 0.1, swa=(wc, ws, np.zeros((2, 1), np.int32), 16))
    assert np.array_equal(o_e, o_s) and np.array_equal(l_e, l_s)
    o_n, l_n = oracle.sparse_attend(q, codes, scales, np.full_like(idx, -1), 0.1,
                                    swa=(wc, ws, np.zeros((2, 1), np.int32), 16))
    assert np.all(o_n == 0) and np.all(np.isneginf(l_n))
