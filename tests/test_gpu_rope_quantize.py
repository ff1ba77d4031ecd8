"""GPU parity of fp8_rope_quantize against the oracle: codes bit-exact.

The rotation is plain fp32 on both sides, operation by operation, so every
code must match.  The one exception is the sign of a NaN that the arithmetic
itself creates (inf - inf, inf * 0): IEEE leaves it open, so where the oracle
writes a NaN code either NaN code is accepted.
"""

import numpy as np
import pytest
import torch

from oracle import quantize as OQ
from oracle import rope as ORO

pytestmark = pytest.mark.gpu


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def roformer_cache(max_pos: int, R: int, base: float = 10000.0) -> torch.Tensor:
    i = np.arange(R // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-2.0 * i / R)[None, :]
    return torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32))


def assert_codes_equal(got: np.ndarray, want: np.ndarray):
    nan_w = (want & 0x7F) == 0x7F
    assert np.array_equal(got[~nan_w], want[~nan_w])
    assert np.all((got[nan_w] & 0x7F) == 0x7F)


def check(gpu, x_pe, cache, pos, neox, scale, x_nope=None, tokens=None):
    out = gpu.fp8_rope_quantize(x_pe, cache.cuda(), pos.cuda(), x_nope=x_nope, is_neox=neox, scale=scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    pe = x_pe if x_pe.dim() == 3 else x_pe.unsqueeze(1)
    sel = slice(None) if tokens is None else torch.as_tensor(tokens)
    dt = OQ.BF16 if x_pe.dtype == torch.bfloat16 else OQ.FP16
    want = ORO.rope_quantize(None if x_nope is None else bits_of(x_nope[sel]), bits_of(pe[sel]), dt,
                             cache.numpy(), pos.numpy()[sel], neox, scale)
    assert_codes_equal(got[sel], want)
    return got


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("scale", [None, 0.37])
def test_mla_query_rows(gpu, neox, scale):
    """q_nope / q_pe as the two parts of one [T, 16, 576] projection output."""
    torch.manual_seed(0)
    T = 300
    q = (torch.randn(T, 16, 576) * 2).to(torch.bfloat16).cuda()
    pos = torch.randint(0, 4096, (T,), dtype=torch.int64)
    check(gpu, q[..., 512:], roformer_cache(4096, 64), pos, neox, scale, x_nope=q[..., :512])


@pytest.mark.parametrize("neox", [True, False])
def test_key_rows_with_a_shared_rope_head(gpu, neox):
    torch.manual_seed(1)
    T = 257
    k_nope = torch.randn(T, 16, 128).to(torch.bfloat16).cuda()
    k_pe = torch.randn(T, 1, 64).to(torch.bfloat16).cuda()
    pos = torch.arange(T, dtype=torch.int64) * 3
    got = check(gpu, k_pe, roformer_cache(1024, 64), pos, neox, 1.5, x_nope=k_nope)
    assert np.array_equal(got[:, 0, 128:], got[:, 15, 128:])


def test_rope_only_rows_fp16_with_wide_rope(gpu):
    torch.manual_seed(2)
    T = 100
    x = (torch.randn(T, 4, 128) * 5).to(torch.float16).cuda()
    pos = torch.randint(0, 100000, (T,), dtype=torch.int64)
    check(gpu, x, roformer_cache(100000, 128, base=1e6), pos, True, None)


def test_out_of_range_positions_write_nan(gpu):
    torch.manual_seed(3)
    T = 40
    q = torch.randn(T, 2, 80).to(torch.bfloat16).cuda()
    pos = torch.randint(0, 64, (T,), dtype=torch.int64)
    pos[[0, 7, 39]] = torch.tensor([-1, 64, 1 << 40])
    got = check(gpu, q[..., 64:], roformer_cache(64, 16), pos, False, None, x_nope=q[..., :64])
    assert np.all(got[[0, 7, 39], :, 64:] == 0x7F)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("neox", [True, False])
def test_every_bit_pattern(gpu, dtype, neox):
    """All 65536 16-bit patterns as rope inputs (inf, NaN, subnormals, overflow)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.int16)
    x = torch.from_numpy(bits).view(dtype).reshape(1024, 1, 64).cuda()
    pos = torch.from_numpy(np.random.default_rng(4).integers(0, 2048, 1024).astype(np.int64))
    check(gpu, x, roformer_cache(2048, 64), pos, neox, 0.25)


def test_into_a_preallocated_strided_output(gpu):
    """Rows written into a slice of a wider buffer; bytes outside the slice untouched."""
    torch.manual_seed(5)
    T, H = 64, 8
    q = torch.randn(T, H, 192).to(torch.bfloat16).cuda()
    buf = torch.full((T, H, 256), 0x55, dtype=torch.uint8, device="cuda")
    out = buf[..., 32:224]
    pos = torch.randint(0, 512, (T,), dtype=torch.int64)
    gpu.fp8_rope_quantize(q[..., 128:], roformer_cache(512, 64).cuda(), pos.cuda(), x_nope=q[..., :128],
                          out=out)
    torch.cuda.synchronize()
    want = ORO.rope_quantize(bits_of(q[..., :128]), bits_of(q[..., 128:]), OQ.BF16,
                             roformer_cache(512, 64).numpy(), pos.numpy(), True, None)
    assert_codes_equal(out.cpu().numpy(), want)
    b = buf.cpu().numpy()
    assert np.all(b[..., :32] == 0x55) and np.all(b[..., 224:] == 0x55)


def test_full_size_mla_queries_sampled(gpu):
    """4096 tokens x 128 heads x (512 + 64): the long-MLA query shape, 48 tokens checked."""
    g = torch.Generator(device="cuda").manual_seed(6)
    T = 4096
    q = torch.randn((T, 128, 576), generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int64)
    tokens = np.sort(np.random.default_rng(7).choice(T, 48, replace=False))
    check(gpu, q[..., 512:], roformer_cache(T, 64), pos, True, None, x_nope=q[..., :512], tokens=tokens)
