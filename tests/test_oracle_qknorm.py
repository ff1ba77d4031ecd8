"""Pins for the oracle's per-head RMS norm + RoPE + e4m3 quantization (CPU only).

The expected codes below are written by hand from the OCP e4m3 bit layout
(sign | 4-bit exponent, bias 7 | 3-bit mantissa): 0.5 = 0x30, 0.75 = 0x34,
1.0 = 0x38, 1.5 = 0x3C, 2.0 = 0x40, 3.0 = 0x44, negatives set bit 7.
"""

import numpy as np
import pytest

from oracle import qknorm as QN
from oracle import quantize as Q

CODE = {0.0: 0x00, 0.5: 0x30, 0.75: 0x34, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 3.0: 0x44}


def code_of(v: float) -> int:
    return CODE[abs(v)] | (0x80 if np.signbit(v) else 0)


def bf16_bits(f) -> np.ndarray:
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def identity_cache(R):
    return np.array([[1.0] * (R // 2) + [0.0] * (R // 2)], dtype=np.float32)


def quarter_cache(R):
    return np.array([[0.0] * (R // 2) + [1.0] * (R // 2)], dtype=np.float32)


W8 = np.array([0.5, 1.0, 1.5, 2.0, 3.0, -3.0, 1.0, -0.5], dtype=np.float32)
SIGNS8 = np.array([1, -1, 1, 1, -1, 1, -1, -1], dtype=np.float32)


@pytest.mark.parametrize("a", [0.75, 3.0, 0.125, 40.0])
def test_equal_magnitude_rows_normalise_to_the_weight(a):
    """|x_i| = a for every i: mean(x^2) = a^2, r = 1/a, y_i = sign_i * w_i
    (fl32(a * fl32(1/a)) rounds back to exactly 1 for these a)."""
    x = bf16_bits((SIGNS8 * a)[None, None, :])
    got = QN.qknorm_rope_quantize(x, Q.BF16, W8, 0.0, identity_cache(2), np.zeros(1, np.int64), 0,
                                  True, None)
    want = np.array([code_of(float(s * w)) for s, w in zip(SIGNS8, W8)], dtype=np.uint8)
    assert np.array_equal(got[0, 0], want)


def test_eps_closed_forms():
    # a row of zeros normalises to zeros (negative zero where the weight is negative)
    x = bf16_bits(np.zeros((1, 2, 8)))
    got = QN.qknorm_rope_quantize(x, Q.BF16, W8, 1e-6, identity_cache(2), np.zeros(1, np.int64), 0, True, None)
    assert np.all(got == np.where(W8 < 0, 0x80, 0x00))
    # |x_i| = 0.75, eps = 0.4375: mean + eps = 1, r = 1, y = x * w; with w = 1, codes of +-0.75
    x = bf16_bits((SIGNS8 * 0.75)[None, None, :])
    got = QN.qknorm_rope_quantize(x, Q.BF16, np.ones(8, np.float32), 0.4375, identity_cache(2),
                                  np.zeros(1, np.int64), 0, True, None)
    assert np.array_equal(got[0, 0], [code_of(float(s * 0.75)) for s in SIGNS8])


@pytest.mark.parametrize("k", [3, -5])
def test_power_of_two_rescaling_leaves_codes_unchanged(k):
    rng = np.random.default_rng(k + 10)
    x = bf16_bits(rng.standard_normal((7, 3, 64)))
    x2 = bf16_bits(Q.widen_to_fp32(x, Q.BF16) * np.float32(2.0 ** k))
    w = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    cache = np.random.default_rng(1).standard_normal((16, 32)).astype(np.float32)
    pos = rng.integers(0, 16, 7)
    a = QN.qknorm_rope_quantize(x, Q.BF16, w, 0.0, cache, pos, 32, True, 0.7)
    b = QN.qknorm_rope_quantize(x2, Q.BF16, w, 0.0, cache, pos, 32, True, 0.7)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", [Q.BF16, Q.FP16])
def test_norm_matches_the_float64_formula(dtype):
    """y = x / sqrt(mean(x^2) + eps) * w in float64, within the three fp32
    roundings (of r, x * r and * w) the oracle takes."""
    rng = np.random.default_rng(3)
    f = (rng.standard_normal((20, 4, 128)) * rng.uniform(0.01, 30, (20, 4, 1))).astype(np.float32)
    bits = bf16_bits(f) if dtype == Q.BF16 else f.astype(np.float16).view(np.uint16)
    w = rng.uniform(-2, 2, 128).astype(np.float32)
    eps = 1e-5
    got = QN.rms_norm_fp32(bits, dtype, w, eps).astype(np.float64)
    x = Q.widen_to_fp32(bits, dtype).astype(np.float64)
    want = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + np.float64(np.float32(eps))) * w
    assert np.all(np.abs(got - want) <= 3.01 * 2.0 ** -24 * np.abs(want) + 1e-45)


@pytest.mark.parametrize("neox", [True, False])
def test_quarter_turn_rotates_the_last_rope_dims_after_the_weight(neox):
    """x = +-1 (r = 1), weight w: y = x * w.  A quarter turn maps each rope
    pair (a, b) to (-b, a) over the LAST R dims only; the weight was applied
    before the rotation, so w of a pair's first dim travels with it."""
    D, R = 8, 4
    signs = SIGNS8
    x = bf16_bits(signs[None, None, :])
    got = QN.qknorm_rope_quantize(x, Q.BF16, W8, 0.0, quarter_cache(R), np.zeros(1, np.int64), R, neox, None)
    y = (signs * W8).astype(np.float64)
    want = y.copy()
    r = y[D - R:]
    if neox:
        want[D - R:] = np.concatenate([-r[R // 2:], r[:R // 2]])
    else:
        rot = np.empty(R)
        rot[0::2], rot[1::2] = -r[1::2], r[0::2]
        want[D - R:] = rot
    assert np.array_equal(got[0, 0], [code_of(float(v)) for v in want])


def test_invalid_positions_write_nan_over_the_rope_dims_only():
    x = bf16_bits((SIGNS8 * 0.75)[None, None, :].repeat(3, axis=0))
    pos = np.array([-1, 0, 5], np.int64)             # cache has one row: 5 is out of range
    got = QN.qknorm_rope_quantize(x, Q.BF16, W8, 0.0, identity_cache(4), pos, 4, True, None)
    nope_want = [code_of(float(s * w)) for s, w in zip(SIGNS8[:4], W8[:4])]
    for t in range(3):
        assert list(got[t, 0, :4]) == nope_want
    assert np.all(got[[0, 2], 0, 4:] == 0x7F)
    assert list(got[1, 0, 4:]) == [code_of(float(s * w)) for s, w in zip(SIGNS8[4:], W8[4:])]


def test_infinite_input_gives_nan_there_and_signed_zeros_elsewhere():
    f = (SIGNS8 * 0.75).astype(np.float32)
    f[2] = np.inf
    got = QN.qknorm_rope_quantize(bf16_bits(f[None, None, :]), Q.BF16, W8, 1e-6, identity_cache(2),
                                  np.zeros(1, np.int64), 0, True, None)[0, 0]
    assert got[2] & 0x7F == 0x7F                          # inf * 0 = NaN
    for i in (0, 1, 3, 4, 5, 6, 7):
        assert got[i] == (0x80 if SIGNS8[i] * W8[i] < 0 else 0x00)


def test_store_rows_hand_placed():
    pages, H, ps, D = 3, 2, 4, 8
    cache = np.full((pages, H, ps, D), 0xEE, np.uint8)
    codes = np.arange(5 * H * D, dtype=np.uint8).reshape(5, H, D)
    slots = np.array([5, -1, 11, 12, 0], np.int64)      # 12 = pages * page_size: out of range
    QN.store_rows(cache, codes, slots)
    want = np.full_like(cache, 0xEE)
    want[1, :, 1, :] = codes[0]                           # slot 5 -> page 1, offset 1
    want[2, :, 3, :] = codes[2]                           # slot 11 -> page 2, offset 3
    want[0, :, 0, :] = codes[4]                           # slot 0 -> page 0, offset 0
    assert np.array_equal(cache, want)
