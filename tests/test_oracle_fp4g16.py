"""Pins of the oracle's FP4 layout with one E4M3 scale per 16 channels of each entry and no
global scale ("FP4 Main KV Cache To Halve Storage Again").

Values whose scale and codes are known by hand, the E4M3 rounding and saturation of the
scale, the E2M1 saturation after a rounded-down scale, zero and subnormal scales, the
per-element error bound of the format, group and nibble placement, and attention over
exactly representable entries against dense fp64 softmax attention."""
import numpy as np
import torch

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _q(x):
    x = np.asarray(x, np.float32)
    return oracle.quantize_fp4_g16(x[None, None] if x.ndim == 1 else x[None])


def _deq(codes, gs):
    B, n, Dh = codes.shape
    idx = np.arange(n, dtype=np.int32)[None, None].repeat(B, 0)
    return oracle.gather_dequant(codes, gs, idx)[:, 0]


def test_exact_group_with_scale_a_power_of_two():
    # amax 12 -> scale 2 exactly (E4M3 0x40); every value is on the E2M1 grid times 2
    vals = np.array([12, 6, -3, 1, 0, 8, -12, 2, 4, -1, 3, 0, 6, -8, 2, 1], np.float32)
    codes, gs = _q(np.concatenate([vals, vals / 4]))
    assert gs[0, 0, 0] == 0x40 and gs[0, 0, 1] == 0x30  # 2.0 and 0.5
    # first byte: channel 0 (12/2 = 6 -> code 7) low nibble, channel 1 (6/2 = 3 -> 5) high
    assert codes[0, 0, 0] == (7 | 5 << 4)
    # channel 2 = -3 -> -1.5 -> code 3 | sign
    assert codes[0, 0, 1] & 15 == (3 | 8)
    assert np.array_equal(_deq(codes, gs)[0, 0], np.concatenate([vals, vals / 4]))


def test_scale_rounds_to_nearest_even_and_values_saturate():
    # amax / 6 = 1.0625 lies halfway between E4M3 1.0 (even) and 1.125: rounds to 1.0, and
    # the largest value, 6.375 / 1.0, saturates to 6
    x = np.zeros(16, np.float32)
    x[3] = 6.375
    x[5] = -2.0
    codes, gs = _q(x)
    assert gs[0, 0, 0] == 0x38
    d = _deq(codes, gs)[0, 0]
    assert d[3] == 6.0 and d[5] == -2.0
    # amax / 6 = 1.07 is nearer 1.125 (0x39)
    x[3] = 6.42
    codes, gs = _q(x)
    assert gs[0, 0, 0] == 0x39
    assert _deq(codes, gs)[0, 0][3] == 6.0 * 1.125


def test_scale_saturates_at_448():
    x = np.zeros(16, np.float32)
    x[0] = 6000.0
    codes, gs = _q(x)
    assert gs[0, 0, 0] == 0x7E
    assert _deq(codes, gs)[0, 0][0] == 6.0 * 448.0


def test_zero_and_subnormal_scales():
    x = np.zeros(32, np.float32)
    x[16] = 6 * 2.0 ** -10          # scale 2^-10 rounds (tie) to E4M3 0 -> the group is zero
    codes, gs = _q(x)
    assert gs[0, 0, 0] == 0 and gs[0, 0, 1] == 0 and np.all(codes == 0)
    x[16] = 6 * 3 * 2.0 ** -10      # scale 1.5 * 2^-9 -> 2 * 2^-9 (subnormal code 2)
    codes, gs = _q(x)
    assert gs[0, 0, 1] == 2
    # 18 * 2^-10 / 2^-8 = 4.5 rounds to the E2M1 value 4
    assert _deq(codes, gs)[0, 0][16] == 4 * 2.0 ** -8


def _half_step(y):
    a = np.abs(y)
    return np.where(a <= 2.0, 0.25, np.where(a <= 4.0, 0.5, 1.0))


def test_error_bound_and_group_placement_random():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(3, 50, 512)).astype(np.float32)
    x[:, :, 37] *= 20.0                         # an outlier channel: only its group's scale grows
    x[1, 7, 128:144] = 0.0                      # an all-zero group
    codes, gs = oracle.quantize_fp4_g16(x)
    deq = _deq(codes, gs)
    sv = np.vectorize(oracle.e4m3_value)(gs.astype(np.int64))            # [3][50][32]
    svc = np.repeat(sv, 16, axis=-1)
    y = np.divide(x, svc, out=np.zeros_like(x), where=svc > 0)
    # within half an E2M1 step of x / s (times s), or clipped at 6 when the scale rounded down
    err = np.abs(deq - x)
    bound = svc * np.where(np.abs(y) > 6.0, np.abs(y) - 6.0, _half_step(y)) + 1e-6 * np.abs(x)
    assert np.all(err <= bound)
    # the scale follows each group's own absmax (1/16 relative rounding of E4M3)
    amax = np.abs(x).reshape(3, 50, 32, 16).max(-1)
    assert np.all(np.abs(sv - amax / 6) <= amax / 6 / 16 + 1e-30)
    assert np.all(gs[1, 7, 8] == 0) and np.all(deq[1, 7, 128:144] == 0)
    # where the outlier is large, only its own group (channels 32..47) has a large scale
    big = np.abs(x[:, :, 37]) >= 12.0
    assert big.sum() > 20
    others = np.delete(sv, 2, axis=-1)
    assert np.all(sv[:, :, 2][big] >= 1.875) and np.all(others[big] < 1.0)


def test_append_rows_at_n0_keep_other_rows():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(2, 5, 64)).astype(np.float32)
    codes, gs = oracle.quantize_fp4_g16(x, n_max=12)
    new = rng.normal(size=(2, 3, 64)).astype(np.float32)
    oracle.quantize_fp4_g16(new, n_max=12, n0=np.array([5, 9], np.int32), codes=codes, gscales=gs)
    c1, g1 = oracle.quantize_fp4_g16(new)
    assert np.array_equal(codes[0, 5:8], c1[0]) and np.array_equal(gs[1, 9:12], g1[1])
    c0, g0 = oracle.quantize_fp4_g16(x)
    assert np.array_equal(codes[:, :5], c0) and np.array_equal(gs[:, :5], g0)


def test_attention_over_exact_entries_is_dense_softmax():
    # entries built on the format's grid (per-group scale times E2M1 values): the dequantised
    # rows equal the fp32 inputs, so sparse attention over all of them is dense attention
    rng = np.random.default_rng(4)
    n, D, Hq = 40, 128, 4
    grid = np.array(E2M1, np.float32)
    sign = rng.choice([-1.0, 1.0], size=(n, D)).astype(np.float32)
    vals = grid[rng.integers(0, 8, size=(n, D))] * sign
    vals.reshape(n, D // 16, 16)[:, :, 0] = 6.0          # amax 6 per group, so x/6 * s is exact
    scale_vals = np.float32(2.0) ** rng.integers(-3, 4, size=(n, D // 16)).astype(np.float32)
    x = (vals.reshape(n, D // 16, 16) * scale_vals[..., None]).reshape(n, D)
    codes, gs = oracle.quantize_fp4_g16(x[None])
    assert np.array_equal(_deq(codes, gs)[0], x)
    q = rng.normal(size=(1, 1, Hq, D)).astype(np.float32)
    idx = rng.permutation(n).astype(np.int32)[None, None]
    out, lse = oracle.sparse_attend(q, codes, gs, idx, 0.05)
    kv = torch.from_numpy(x.astype(np.float64))
    logits = 0.05 * torch.from_numpy(q[0, 0].astype(np.float64)) @ kv.T
    ref = torch.softmax(logits, dim=-1) @ kv
    assert np.allclose(out[0, 0], ref.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[0, 0], torch.logsumexp(logits, -1).numpy(), rtol=1e-12, atol=1e-12)
