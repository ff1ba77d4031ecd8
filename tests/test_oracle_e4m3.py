"""Pins for the oracle's e4m3fn codec (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(v):
    t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_matches_library_on_all_codes():
    ours = e4m3.decode_table()
    lib = torch_decode_all()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x7E, 448.0), (0x7D, 416.0),
    (0x81, -(2.0 ** -9)), (0xB8, -1.0), (0xFE, -448.0),
])
def test_decode_hand_values(code, value):
    # values of the OCP E4M3 table (bias 7, subnormal step 2^-9, max 448)
    assert e4m3.decode(np.array([code], np.uint8))[0] == value


def test_decode_structure():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0..126 must be strictly increasing"
    assert np.array_equal(t[0x80:0xFF], -pos)
    assert np.signbit(t[0x80]) and t[0x80] == 0.0


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)


def _grid_sweep():
    t = e4m3.decode_table()
    pos = t[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2
    pts = [pos, mids]
    for f in (1 - 2.0 ** -20, 1 + 2.0 ** -20):
        pts += [mids * f, pos * f]
    rng = np.random.default_rng(0)
    pts.append(np.exp(rng.uniform(np.log(2.0 ** -14), np.log(460.0), 200_000)))
    v = np.concatenate(pts)
    v = v[v <= 464.0].astype(np.float32)
    return np.concatenate([v, -v, np.float32([0.0, -0.0, 2.0 ** -140, -(2.0 ** -140)])])


def test_encode_matches_library_rne_below_saturation():
    v = _grid_sweep()
    ours = e4m3.encode(v)
    lib = torch_encode(v)
    bad = np.nonzero(ours != lib)[0]
    assert bad.size == 0, f"first mismatches: {v[bad[:5]]} ours {ours[bad[:5]]} lib {lib[bad[:5]]}"


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),             # tie between 1.0 and 1.125 -> even (1.0)
    (1.1875, 0x3A),             # tie between 1.125 and 1.25 -> even (1.25)
    (3 * 2.0 ** -10, 0x02),     # subnormal tie -> even (2 * 2^-9)
    (2.0 ** -10, 0x00),         # half the smallest subnormal -> 0
    (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (480.0, 0x7E),
    (1e9, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE), (-1e30, 0xFE),
    (-0.0, 0x80), (np.nan, 0x7F),
])
def test_encode_hand_table(value, code):
    assert int(e4m3.encode(np.array([value], np.float64))[0]) == code
