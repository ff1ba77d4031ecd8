"""fp8_quantize on the GPU vs the oracle: bit-exact bytes."""

import numpy as np
import pytest
import torch

from oracle import quantize as OQ
import workloads as W
from helpers import bf16_dev, dev, host, workload

pytestmark = pytest.mark.gpu

SCALES = [None, 0.5, 0.25, 2.0] + [float(s) for s in np.random.default_rng(77).uniform(0.1, 4.0, 5)]


def all_patterns(dtype):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16 if dtype == OQ.BF16 else torch.float16)
    return bits, t.cuda()


@pytest.mark.parametrize("dtype", [OQ.BF16, OQ.FP16])
@pytest.mark.parametrize("scale", SCALES)
def test_exhaustive_bit_patterns(gpu, dtype, scale):
    bits, x = all_patterns(dtype)
    got = host(gpu.fp8_quantize(x.reshape(256, 256), scale)).reshape(-1)
    ref = OQ.quantize(bits, dtype, scale)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (f"{bad.size} mismatches, first bits {bits[bad[:8]]} "
                           f"gpu {got[bad[:8]]} oracle {ref[bad[:8]]}")


@pytest.mark.parametrize("shape", [(1,), (7,), (3, 5), (33, 129), (2, 3, 1000), (1, 1, 8), (0, 16)])
def test_ragged_shapes(gpu, shape):
    rng = np.random.default_rng(len(shape))
    x = W.bf16_bits(rng.standard_normal(shape).astype(np.float32) * 7)
    got = host(gpu.fp8_quantize(bf16_dev(x), 0.37))
    assert np.array_equal(got, OQ.quantize(x, OQ.BF16, 0.37))


def test_strided_rows_and_output(gpu):
    rng = np.random.default_rng(5)
    full = W.bf16_bits(rng.standard_normal((6, 40, 264)).astype(np.float32) * 3)
    xt = bf16_dev(full)[:, :, :256]                 # row stride 264, 8-aligned -> vector path
    out = torch.zeros((6, 40, 300), dtype=torch.uint8, device="cuda")[:, :, :256]
    gpu.fp8_quantize(xt, 1.5, out=out)
    assert np.array_equal(host(out), OQ.quantize(full[:, :, :256], OQ.BF16, 1.5))
    xs = bf16_dev(full)[:, :, 3:200]                # unaligned start, odd width -> scalar path
    got = host(gpu.fp8_quantize(xs, None))
    assert np.array_equal(got, OQ.quantize(full[:, :, 3:200], OQ.BF16, None))


def test_rejects_non_flattenable(gpu):
    x = torch.zeros((4, 6, 8), dtype=torch.bfloat16, device="cuda")[:, :3, :]
    with pytest.raises(ValueError):
        gpu.fp8_quantize(x)
    with pytest.raises(ValueError):
        gpu.fp8_quantize(torch.zeros(8, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("n", [2, 3, 5])
def test_full_size_workload_queries(gpu, n):
    """Q and idx_q of the 8k / 32k prefill and the decode workload, all bytes."""
    wl = workload(n)
    for bits, s in ((wl.q_bf16, wl.q_scale), (wl.idx_q_bf16, wl.idx_q_scale)):
        got = host(gpu.fp8_quantize(bf16_dev(bits), s))
        assert np.array_equal(got, OQ.quantize(bits, OQ.BF16, s))


def test_full_size_mla_queries_sampled(gpu):
    """Q of the long MLA workload ([4096, 128, 576] bf16), every 61st token checked."""
    wl = workload(4)
    got = host(gpu.fp8_quantize(bf16_dev(wl.q_bf16), wl.q_scale))
    rows = np.arange(0, wl.q_bf16.shape[0], 61)
    assert np.array_equal(got[rows], OQ.quantize(wl.q_bf16[rows], OQ.BF16, wl.q_scale))


def test_mla_tiny_queries(gpu):
    wl = workload(1)
    got = host(gpu.fp8_quantize(bf16_dev(wl.q_bf16), wl.q_scale))
    assert np.array_equal(got, OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale))


# ---------------------------------------------------------------- fp8_quantize_pair
@pytest.mark.parametrize("dtype", [OQ.BF16, OQ.FP16])
@pytest.mark.parametrize("s0,s1", [(None, None), (0.37, None), (None, 2.0), (0.25, 3.3)])
def test_pair_every_bit_pattern(gpu, dtype, s0, s1):
    """All 65536 patterns as the first tensor, a random second tensor of a
    different size: both bit-exact against the oracle, each with its own scale."""
    bits, x0 = all_patterns(dtype)
    rng = np.random.default_rng(9)
    f = rng.standard_normal(8 * 1237).astype(np.float32) * 50
    b1 = W.bf16_bits(f) if dtype == OQ.BF16 else f.astype(np.float16).view(np.uint16)
    x1 = torch.from_numpy(b1.view(np.int16)).view(x0.dtype).cuda()
    g0, g1 = gpu.fp8_quantize_pair(x0.reshape(256, 256), s0, x1, s1)
    assert np.array_equal(host(g0).reshape(-1), OQ.quantize(bits, dtype, s0))
    assert np.array_equal(host(g1), OQ.quantize(b1, dtype, s1))


@pytest.mark.parametrize("n", [2, 5])
def test_pair_equals_two_single_calls_on_workload_queries(gpu, n):
    """Q and idx_q of the 8k prefill and the decode workload: the pair launch
    writes the bytes of two fp8_quantize calls, and the oracle's."""
    wl = workload(n)
    q, iq = bf16_dev(wl.q_bf16), bf16_dev(wl.idx_q_bf16)
    g0, g1 = gpu.fp8_quantize_pair(q, wl.q_scale, iq, wl.idx_q_scale)
    assert torch.equal(g0, gpu.fp8_quantize(q, wl.q_scale))
    assert torch.equal(g1, gpu.fp8_quantize(iq, wl.idx_q_scale))
    assert np.array_equal(host(g0), OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale))
    assert np.array_equal(host(g1), OQ.quantize(wl.idx_q_bf16, OQ.BF16, wl.idx_q_scale))


def test_pair_edge_sizes(gpu):
    """An empty tensor on either side, a single chunk, and tensors smaller than
    one wave; bytes around the outputs untouched."""
    rng = np.random.default_rng(10)
    for n0, n1 in ((0, 64), (8, 0), (8, 8), (24, 4096), (4096 * 8 + 8, 16)):
        b0 = W.bf16_bits(rng.standard_normal(n0).astype(np.float32))
        b1 = W.bf16_bits(rng.standard_normal(n1).astype(np.float32))
        buf = torch.full((n0 + n1 + 64,), 0x5A, dtype=torch.uint8, device="cuda")
        o0, o1 = buf[16:16 + n0], buf[32 + n0:32 + n0 + n1]
        gpu.fp8_quantize_pair(bf16_dev(b0), 1.25, bf16_dev(b1), None, out0=o0, out1=o1)
        assert np.array_equal(host(o0), OQ.quantize(b0, OQ.BF16, 1.25))
        assert np.array_equal(host(o1), OQ.quantize(b1, OQ.BF16, None))
        h = host(buf)
        assert np.all(h[:16] == 0x5A) and np.all(h[16 + n0:32 + n0] == 0x5A) and np.all(h[32 + n0 + n1:] == 0x5A)
