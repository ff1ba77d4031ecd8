"""Pins for the oracle's fused RoPE + e4m3 quantization (CPU only)."""

import numpy as np
import pytest

from oracle import quantize as Q
from oracle import rope as RO


def bf16_bits(f) -> np.ndarray:
    """bf16 bit patterns of fp32 values, rounded to nearest even."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def widen(bits) -> np.ndarray:
    return Q.widen_to_fp32(bits, Q.BF16)


def roformer_cache(max_pos: int, R: int, base: float = 10000.0) -> np.ndarray:
    """cos ++ sin of p * base^(-2i/R), rounded to fp32 (RoFormer's angles)."""
    i = np.arange(R // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / R)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def inputs(seed, T=6, H=3, nope=16, R=8):
    rng = np.random.default_rng(seed)
    return (bf16_bits(rng.standard_normal((T, H, nope)) * 2),
            bf16_bits(rng.standard_normal((T, H, R)) * 2))


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_position_zero_is_plain_quantization(neox, scale):
    nope, pe = inputs(1)
    cache = roformer_cache(4, pe.shape[-1])           # row 0: cos 1, sin 0
    got = RO.rope_quantize(nope, pe, Q.BF16, cache, np.zeros(nope.shape[0], np.int64), neox, scale)
    want = np.concatenate([Q.quantize(nope, Q.BF16, scale), Q.quantize(pe, Q.BF16, scale)], axis=-1)
    assert np.array_equal(got, want)


def turn_cache(R, cos, sin):
    return np.array([[cos] * (R // 2) + [sin] * (R // 2)], dtype=np.float32)


@pytest.mark.parametrize("scale", [None, 2.0])
def test_quarter_and_half_turns(scale):
    """cos 0 / sin 1: each pair (a, b) -> (-b, a).  cos -1 / sin 0: x -> -x."""
    _, pe = inputs(2)
    T, H, R = pe.shape
    x = widen(pe)
    pos = np.zeros(T, np.int64)
    # rotate-half pairs dim i with dim i + R/2
    want = np.concatenate([-x[..., R // 2:], x[..., :R // 2]], axis=-1)
    got = RO.rope_quantize(None, pe, Q.BF16, turn_cache(R, 0.0, 1.0), pos, True, scale)
    assert np.array_equal(got, Q.quantize(bf16_bits(want), Q.BF16, scale))
    # interleaved pairs dims 2i and 2i + 1
    want = np.empty_like(x)
    want[..., 0::2], want[..., 1::2] = -x[..., 1::2], x[..., 0::2]
    got = RO.rope_quantize(None, pe, Q.BF16, turn_cache(R, 0.0, 1.0), pos, False, scale)
    assert np.array_equal(got, Q.quantize(bf16_bits(want), Q.BF16, scale))
    for neox in (True, False):
        got = RO.rope_quantize(None, pe, Q.BF16, turn_cache(R, -1.0, 0.0), pos, neox, scale)
        assert np.array_equal(got, Q.quantize(bf16_bits(-x), Q.BF16, scale))


@pytest.mark.parametrize("neox", [True, False])
def test_rotation_matches_complex_multiplication(neox):
    rng = np.random.default_rng(3)
    T, H, R = 64, 4, 64
    x = widen(bf16_bits(rng.standard_normal((T, H, R)) * 3))
    cache = roformer_cache(4096, R)
    pos = rng.integers(0, 4096, T)
    got = RO.rope_fp32(x, cache, pos, neox).astype(np.float64)
    xd = x.astype(np.float64)
    a, b = (xd[..., :R // 2], xd[..., R // 2:]) if neox else (xd[..., 0::2], xd[..., 1::2])
    cs = cache[pos].astype(np.float64)
    w = (cs[:, None, :R // 2] + 1j * cs[:, None, R // 2:])
    z = (a + 1j * b) * w
    ga, gb = (got[..., :R // 2], got[..., R // 2:]) if neox else (got[..., 0::2], got[..., 1::2])
    bound = 3 * 2.0 ** -24 * (np.abs(a) + np.abs(b)) * np.abs(w) + 1e-45
    assert np.all(np.abs(ga - z.real) <= bound)
    assert np.all(np.abs(gb - z.imag) <= bound)
    # and the rotation keeps each pair's length (|cos + i sin| = 1 to fp32 precision)
    assert np.allclose(np.abs(ga + 1j * gb), np.abs(a + 1j * b), rtol=1e-6, atol=1e-30)


def test_shared_rope_head_is_broadcast():
    nope, pe = inputs(4, H=3)
    shared = pe[:, :1]
    cache = roformer_cache(64, pe.shape[-1])
    pos = np.arange(6) * 7
    got = RO.rope_quantize(nope, shared, Q.BF16, cache, pos, True, 0.7)
    full = RO.rope_quantize(nope, np.repeat(shared, 3, axis=1), Q.BF16, cache, pos, True, 0.7)
    assert np.array_equal(got, full)
    assert np.array_equal(got[:, 0, 16:], got[:, 2, 16:])


def test_out_of_range_positions_write_nan_codes():
    nope, pe = inputs(5)
    cache = roformer_cache(10, pe.shape[-1])
    pos = np.array([0, -1, 3, 10, 9, 1000])
    got = RO.rope_quantize(nope, pe, Q.BF16, cache, pos, False, None)
    bad = np.array([False, True, False, True, False, True])
    assert np.all(got[bad][..., 16:] == RO.NAN_CODE)
    assert np.array_equal(got[..., :16], Q.quantize(nope, Q.BF16, None))
    ok = RO.rope_quantize(nope[~bad], pe[~bad], Q.BF16, cache, pos[~bad], False, None)
    assert np.array_equal(got[~bad], ok)
