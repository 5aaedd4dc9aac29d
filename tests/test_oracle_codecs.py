"""Pins of the oracle's number formats (E2M1 main KV, E4M3 indexer) and quantisers.

E2M1 and E4M3 are fixed by their bit-field definitions ("FP4 Main KV Cache To Halve
Storage Again" in the paper notes; 3.5 of the Chinese reading: E2M1 values, E4M3 scales).
The expected tables here are written from the format definitions and from torch's own
float8_e4m3fn conversion, not from the oracle's code.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

# The eight E2M1 magnitudes, in code order (format definition: 1 sign, 2 exponent bits
# with bias 1, 1 mantissa bit, exponent 0 subnormal).
E2M1_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    for code in range(16):
        mag = E2M1_MAGS[code & 7]
        v = oracle.e2m1_value(code)
        assert v == (-mag if code & 8 else mag)
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)


def test_e2m1_roundtrip_all_codes():
    for code in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(code)) == code


@pytest.mark.parametrize("y,code", [
    (0.25, 0), (0.2500001, 1), (0.75, 2), (0.7499999, 1), (1.25, 2), (1.2500001, 3), (1.75, 4),
    (2.5, 4), (2.5000002, 5), (3.5, 6), (3.4999998, 5), (5.0, 6), (5.0000005, 7), (6.5, 7), (1e30, 7),
    (float("inf"), 7), (-0.1, 8), (-0.0, 8), (0.0, 0), (-6.0, 15), (float("-inf"), 15), (-3.5, 14),
])
def test_e2m1_ties_and_saturation(y, code):
    # Round to nearest, ties to the even code; saturate to 6; sign kept (also for -0).
    assert oracle.e2m1_encode(np.float32(y)) == code


def _e2m1_threshold_rule(a):
    # Independent statement of RNE-even for E2M1 as decision thresholds on |y|.
    if a <= 0.25: return 0
    if a < 0.75: return 1
    if a <= 1.25: return 2
    if a < 1.75: return 3
    if a <= 2.5: return 4
    if a < 3.5: return 5
    if a <= 5.0: return 6
    return 7


def test_e2m1_matches_threshold_rule():
    rng = np.random.default_rng(0)
    ys = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-7, 7, 0.125)]).astype(np.float32)
    for y in ys:
        expect = _e2m1_threshold_rule(abs(float(y))) | (8 if np.signbit(y) else 0)
        assert oracle.e2m1_encode(y) == expect, y


def test_fp4_all_bytes_repack():
    # Every byte unpacks to two codes and repacks to itself (scale 1, given).
    D = 512
    bytes_ = np.arange(256, dtype=np.uint8)
    x = np.zeros((1, 1, D), np.float32)
    for i, byte in enumerate(bytes_):
        x[0, 0, 2 * i] = E2M1_MAGS[byte & 7] * (-1 if byte & 8 else 1)
        x[0, 0, 2 * i + 1] = E2M1_MAGS[(byte >> 4) & 7] * (-1 if byte & 128 else 1)
    # -0 must keep its sign bit
    x[0, 0, 2 * 8] = -0.0
    x[0, 0, 2 * 128 + 1] = -0.0
    codes, _ = oracle.quantize_fp4(x, scales=np.ones((1, D), np.float32))
    assert np.array_equal(codes[0, 0], bytes_)


def test_fp4_scale_absmax_maps_to_six():
    wl = workloads.workload("full64k", N=256)
    x = wl.main_kv(0)[None]
    codes, s = oracle.quantize_fp4(x)
    amax = np.abs(x[0]).max(axis=0)
    assert np.array_equal(s[0], (amax / np.float32(6)).astype(np.float32))
    t_max = np.abs(x[0]).argmax(axis=0)
    for c in range(x.shape[-1]):
        byte = codes[0, t_max[c], c // 2]
        code = (byte >> 4) if c & 1 else (byte & 15)
        assert code & 7 == 7


def test_fp4_power_of_two_channel_invariance():
    # Scaling one channel by 2^k leaves its codes unchanged and scales s by exactly 2^k.
    wl = workloads.workload("tiny", N=64)
    x = wl.main_kv(0)[None].copy()
    codes0, s0 = oracle.quantize_fp4(x)
    for k, ch in [(3, 5), (-4, 17), (10, 100)]:
        y = x.copy()
        y[..., ch] *= np.float32(2.0 ** k)
        codes1, s1 = oracle.quantize_fp4(y)
        assert np.array_equal(codes0, codes1)
        assert s1[0, ch] == np.float32(s0[0, ch] * 2.0 ** k)


def test_fp4_zero_channel():
    x = np.zeros((1, 4, 32), np.float32)
    x[0, :, 1] = 1.0
    codes, s = oracle.quantize_fp4(x)
    assert s[0, 0] == 0 and s[0, 1] == np.float32(1 / 6)
    assert np.all(codes[0, :, 0] & 15 == 0)


def test_e4m3_table_matches_torch():
    raw = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for code in range(256):
        v = oracle.e4m3_value(code)
        if code in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(raw[code])
        else:
            assert v == raw[code], code
            assert math.copysign(1.0, v) == math.copysign(1.0, raw[code])


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    ys = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 100, 4000), rng.uniform(-448, 448, 4000),
        rng.uniform(-0.02, 0.02, 4000),
    ]).astype(np.float32)
    # midpoints between consecutive finite magnitudes exercise ties-to-even
    mags = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    ys = np.concatenate([ys, mids, -mids])
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(y) for y in ys], np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("y,code", [
    (448.0, 0x7E), (449.0, 0x7E), (500.0, 0x7E), (1e9, 0x7E), (float("inf"), 0x7E), (-1e9, 0xFE),
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (-0.0, 0x80), (2.0 ** -9, 0x01),
])
def test_e4m3_saturation_and_subnormal_ties(y, code):
    assert oracle.e4m3_encode(np.float32(y)) == code


def test_fp8_quantize_per_token():
    wl = workloads.workload("full64k", N=512)
    k = wl.index_keys(0)[None]
    codes, s = oracle.quantize_fp8(k)
    amax = np.abs(k[0]).max(axis=1)
    assert np.array_equal(s[0], (amax / np.float32(448)).astype(np.float32))
    # the absmax element of each row lands on +-448
    jmax = np.abs(k[0]).argmax(axis=1)
    assert np.all(codes[0, np.arange(512), jmax] & 0x7F == 0x7E)
    # the codes are E4M3 of fl32(x / s), checked against torch's conversion
    y = (k[0] / s[0][:, None]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[0], ref)


def test_fp4_append_equals_one_shot():
    # Quantising rows [0, N) with given scales == rows [0, Nc) then appending [Nc, N).
    wl = workloads.workload("full64k", N=96)
    x = wl.main_kv(0)[None]
    _, s = oracle.quantize_fp4(x)
    full, _ = oracle.quantize_fp4(x, scales=s)
    part = np.zeros_like(full)
    oracle.quantize_fp4(x[:, :60], n_max=96, scales=s, codes=part)
    oracle.quantize_fp4(x[:, 60:], n_max=96, n0=np.array([60], np.int32), scales=s, codes=part)
    assert np.array_equal(full, part)


def test_gather_dequant_values():
    wl = workloads.workload("tiny", N=64)
    x = wl.main_kv(0)[None]
    codes, s = oracle.quantize_fp4(x)
    idx = np.array([[[5, -1, 63, 0]]], np.int32)
    g = oracle.gather_dequant(codes, s, idx)
    lo = codes[0] & 15
    hi = codes[0] >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(64, -1)
    table = np.array(E2M1_MAGS + [-m for m in E2M1_MAGS], np.float64)
    deq = (table[nib] * s[0].astype(np.float64)).astype(np.float32)
    assert np.array_equal(g[0, 0, 0], deq[5])
    assert np.all(g[0, 0, 1] == 0)
    assert np.array_equal(g[0, 0, 2], deq[63])
    assert np.array_equal(g[0, 0, 3], deq[0])
    # dequantised values stay within half a code step of the input (plus saturation: none here)
    assert np.all(np.abs(deq - x[0]) <= s[0] * 1.0 + 1e-7)
