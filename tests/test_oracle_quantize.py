"""Pins for the oracle's per-tensor quantizer (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import quantize as Q

SCALES = [None, 0.5, 0.25, 2.0, 0.1234567, 3.7]


def all_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def library_quantize(bits, dtype, scale):
    """torch's fp32 multiply and e4m3fn cast; NaN where torch leaves the format."""
    if dtype == Q.BF16:
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    else:
        x = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float32)
    if scale is not None:
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32)
        x = x * inv
    return x.numpy(), x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("dtype", [Q.BF16, Q.FP16])
@pytest.mark.parametrize("scale", SCALES)
def test_exhaustive_vs_library(dtype, scale):
    bits = all_bits()
    ours = Q.quantize(bits, dtype, scale)
    v, lib = library_quantize(bits, dtype, scale)
    ok = np.isfinite(v) & (np.abs(v) <= 464.0)
    assert np.array_equal(ours[ok], lib[ok])
    # outside the library's range the oracle saturates / maps NaN by its reading
    sat = np.isfinite(v) & (np.abs(v) > 464.0) | np.isinf(v)
    assert np.all((ours[sat] & 0x7F) == 0x7E)
    assert np.array_equal(ours[sat] >> 7, np.signbit(v[sat]).astype(np.uint8))
    nan = np.isnan(v)
    assert np.all((ours[nan] & 0x7F) == 0x7F)


def test_none_equals_unit_scale():
    bits = all_bits()
    for dt in (Q.BF16, Q.FP16):
        assert np.array_equal(Q.quantize(bits, dt, None), Q.quantize(bits, dt, 1.0))


def test_power_of_two_scale_shifts_exactly():
    # x / 2 of an e4m3-exact value, well inside the normal range, is e4m3-exact
    bits = all_bits()
    x = Q.widen_to_fp32(bits, Q.BF16)
    sel = np.isfinite(x) & (np.abs(x) >= 2.0 ** -4) & (np.abs(x) <= 224.0)
    a = Q.quantize(bits[sel], Q.BF16, 2.0)
    b = Q.quantize(bits[sel], Q.BF16, None)
    from oracle import e4m3
    da, db = e4m3.decode(a), e4m3.decode(b)
    # rounding x/2 on the grid equals half of rounding x (grid scales with the binade)
    assert np.array_equal(da * 2.0, db)


def test_reciprocal_is_rounded_once_in_fp32():
    s = 0.1234567
    inv = Q.scale_inv_fp32(s)
    assert inv.dtype == np.float32
    assert inv == np.float32(1.0) / np.float32(s)
