"""Pins of the oracle's 4-bit indexer variant ("FP4 Main KV Cache To Halve Storage Again":
the indexer queries and keys are 4-bit): E2M1 keys with one absmax/6 scale per row and the
query quantised the same way per (token, head).

The row quantiser is checked against the per-channel FP4 quantiser (already pinned) on the
transposed problem, on hand-worked values, scaling by powers of two and zero rows; the
score against an einsum of operands decoded through the E2M1 table written from the
format's definition."""
import numpy as np

import oracle

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack(codes):
    lo, hi = codes & 15, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], -1).astype(np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1[c & 7]


def test_rows_match_the_per_channel_quantiser_on_the_transpose():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(3, 40, 64)).astype(np.float32)
    x[1, 5] = 0.0
    codes, s = oracle.quantize_fp4_rows(x)
    for b in range(3):
        ct, st = oracle.quantize_fp4(np.ascontiguousarray(x[b].T)[None])   # rows become channels
        assert np.array_equal(st[0], s[b])
        assert np.array_equal(_unpack(ct[0]).T, _unpack(codes[b]))


def test_hand_worked_row_and_scaling():
    x = np.array([[[3.0, -1.5, 0.75, 0.0, 1.0, -3.0, 2.0, 0.5]]], np.float32)   # absmax 3 -> s = 0.5
    codes, s = oracle.quantize_fp4_rows(x)
    assert s[0, 0] == 0.5
    assert codes[0, 0, 0] == (7 | (5 | 8) << 4)          # 6 and -3 (dims 0, 1: low, high nibble)
    assert np.array_equal(_unpack(codes)[0, 0] * 0.5, x[0, 0])
    c2, s2 = oracle.quantize_fp4_rows(x * 2.0 ** -7)
    assert np.array_equal(c2, codes) and s2[0, 0] == 0.5 * 2.0 ** -7
    z, sz = oracle.quantize_fp4_rows(np.zeros((1, 2, 8), np.float32))
    assert np.all(z == 0) and np.all(sz == 0)


def test_score_is_the_einsum_of_decoded_operands():
    rng = np.random.default_rng(1)
    B, T, H, dk, n = 2, 3, 32, 64, 70
    k = rng.normal(size=(B, n, dk)).astype(np.float32)
    q = rng.normal(size=(B, T, H, dk)).astype(np.float32)
    w = rng.random((B, T, H)).astype(np.float32)
    kc, ks = oracle.quantize_fp4_rows(k)
    qc, qs = oracle.quantize_fp4_rows(q.reshape(1, B * T * H, dk))      # per (token, head), same rule
    kd = _unpack(kc) * ks[..., None].astype(np.float64)
    qd = (_unpack(qc) * qs[..., None].astype(np.float64)).reshape(B, T, H, dk)
    ref = np.einsum("bth,bthd,bnd->btn", w.astype(np.float64), qd, kd)
    nk = np.array([70, 33], np.int32)
    got = oracle.index_score(oracle.PREC_FP4, q, w, kc, ks, nk)
    vis = np.arange(n)[None, None, :] < nk[:, None, None]
    assert np.all(np.isneginf(got[~np.broadcast_to(vis, got.shape)]))
    assert np.allclose(got[np.broadcast_to(vis, got.shape)], ref[np.broadcast_to(vis, ref.shape)], rtol=1e-12,
                       atol=1e-9)
