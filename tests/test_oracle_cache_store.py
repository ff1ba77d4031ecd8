"""Pins for the oracle's paged fp8 cache store (CPU only)."""

import numpy as np
import pytest

from oracle import cache_store as CS
from oracle import e4m3 as E
from oracle import quantize as Q


def bf16_of(values) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly (checked)."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f)
    return bits


def test_hand_placed_layout():
    """Tiny layout with every byte placed by hand.

    pages=2, heads=2, page_size=3, row = dim 2 + dim2 1.  Slots: token 0 -> 4
    (page 1, offset 1), token 1 -> -1 (padding), token 2 -> 0 (page 0, offset 0),
    token 3 -> 6 (= pages * page_size, out of range).  Scale 2.0, so each code
    is that of x / 2 in the OCP e4m3 layout (sign, 4 exponent bits with bias 7,
    3 mantissa bits): 1.0 = 0x38, 2.0 = 0x40, 0.5 = 0x30, 3.0 = 0x44,
    -1.0 = 0xB8, 448 = 0x7E, 1.5 = 0x3C, 0 = 0x00.
    """
    x = np.array([[[2.0, 4.0], [6.0, -2.0]],
                  [[3.0, 3.0], [3.0, 3.0]],
                  [[3.0, 0.0], [1.0, 2.0]],
                  [[8.0, 8.0], [8.0, 8.0]]])
    x2 = np.array([[[1.0], [896.0]],
                   [[3.0], [3.0]],
                   [[-2.0], [6.0]],
                   [[8.0], [8.0]]])
    cache = np.full((2, 2, 3, 3), 0x11, dtype=np.uint8)
    got = CS.cache_store(cache, bf16_of(x), Q.BF16, np.array([4, -1, 0, 6]), 2.0, bf16_of(x2))
    want = np.full((2, 2, 3, 3), 0x11, dtype=np.uint8)
    want[1, 0, 1] = [0x38, 0x40, 0x30]
    want[1, 1, 1] = [0x44, 0xB8, 0x7E]
    want[0, 0, 0] = [0x3C, 0x00, 0xB8]
    want[0, 1, 0] = [0x30, 0x38, 0x44]
    assert np.array_equal(got, want)
    assert np.all(cache == 0x11), "the input cache must not be modified"


@pytest.mark.parametrize("dtype", [Q.BF16, Q.FP16])
@pytest.mark.parametrize("scale", [None, 0.37, 3.0])
def test_read_back_and_untouched(dtype, scale):
    rng = np.random.default_rng(11)
    pages, heads, page_size, dim = 5, 2, 8, 16
    n = 23
    slots = rng.permutation(pages * page_size)[:n].astype(np.int64)
    slots[[3, 9]] = -1
    f = (rng.standard_normal((n, heads, dim)) * 3).astype(np.float32)
    bits = bf16_of((f.view(np.uint32) & 0xFFFF0000).view(np.float32)) if dtype == Q.BF16 else \
        f.astype(np.float16).view(np.uint16)
    cache = rng.integers(0, 256, (pages, heads, page_size, dim), dtype=np.uint8)
    got = CS.cache_store(cache, bits, dtype, slots, scale)
    want_rows = Q.quantize(bits, dtype, scale)
    touched = np.zeros((pages, page_size), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        p, o = divmod(int(s), page_size)
        touched[p, o] = True
        assert np.array_equal(got[p, :, o], want_rows[i])
    keep = ~touched
    assert np.array_equal(got.transpose(0, 2, 1, 3)[keep], cache.transpose(0, 2, 1, 3)[keep])


@pytest.mark.parametrize("scale", [0.25, 1.0, 8.0])
def test_round_trip_exact_values(scale):
    """x = scale * (an e4m3 value) is stored as that value's code: decode * scale == x."""
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = rng.choice(finite, (40, 1, 32))
    x = E.decode(codes) * scale
    cache = np.zeros((40, 1, 1, 32), dtype=np.uint8)       # flat [S, row] layout: page_size 1
    got = CS.cache_store(cache, bf16_of(x), Q.BF16, np.arange(40), scale)
    assert np.array_equal(E.decode(got[:, 0, 0]) * scale, x[:, 0])
    # -0.0 keeps its sign; every other code round-trips to itself
    assert np.array_equal(got[:, 0, 0], codes[:, 0])
