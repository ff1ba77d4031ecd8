"""GPU parity of fp8_cache_store against the oracle: every cache byte bit-exact."""

import numpy as np
import pytest
import torch

from oracle import cache_store as OCS
from oracle import quantize as OQ

pytestmark = pytest.mark.gpu


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_and_compare(gpu, x, slots, cache, scale, x2=None):
    """Store through the C ABI and compare the whole cache with the oracle."""
    dt = OQ.BF16 if x.dtype == torch.bfloat16 else OQ.FP16
    before = cache.cpu().numpy()
    xb = bits_of(x if x.dim() == 3 else x.unsqueeze(1))
    x2b = None if x2 is None else bits_of(x2 if x2.dim() == 3 else x2.unsqueeze(1))
    gpu.fp8_cache_store(x, slots, cache, scale=scale, x2=x2)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    if before.ndim == 2:
        shape4 = (before.shape[0], 1, 1, before.shape[1])
    elif before.ndim == 3:
        shape4 = (before.shape[0], 1, before.shape[1], before.shape[2])
    else:
        shape4 = before.shape
    want = OCS.cache_store(before.reshape(shape4), xb, dt, slots.cpu().numpy(), scale, x2b)
    assert np.array_equal(got.reshape(shape4), want)


def random_cache(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(0, 256, shape, generator=g, dtype=torch.uint8).cuda()


def random_slots(n, n_slots, seed, pad=()):
    rng = np.random.default_rng(seed)
    s = rng.permutation(n_slots)[:n].astype(np.int64)
    for i in pad:
        s[i] = -1
    return s


def test_block_kv_cache_from_fused_projection(gpu):
    """K part of a fused QKV projection (token stride 20*128) into [pages, 2, 128, 128]."""
    torch.manual_seed(0)
    n, pages = 700, 6
    qkv = (torch.randn(n, 20 * 128) * 3).to(torch.bfloat16).cuda()
    k = qkv[:, 16 * 128:18 * 128].view(n, 2, 128)
    s = random_slots(n, pages * 128, 1, pad=(0, 5, 699))
    s[7] = pages * 128 + 3                     # beyond the cache: skipped
    run_and_compare(gpu, k, torch.from_numpy(s).cuda(), random_cache((pages, 2, 128, 128), 2), 0.37)


@pytest.mark.parametrize("scale", [None, 2.5])
def test_index_k_cache_fp16(gpu, scale):
    torch.manual_seed(1)
    n, pages = 333, 4
    x = (torch.randn(n, 128) * 4).to(torch.float16).cuda()
    s = random_slots(n, pages * 128, 3, pad=(10,))
    run_and_compare(gpu, x, torch.from_numpy(s).cuda(), random_cache((pages, 128, 128), 4), scale)


def test_mla_latent_and_rope_pack(gpu):
    """kv_a [N, 512] + k_pe [N, 64] (a strided view) into flat [S, 576] rows."""
    torch.manual_seed(2)
    n, S = 257, 1000
    kv_a = torch.randn(n, 512).to(torch.bfloat16).cuda()
    pe_src = torch.randn(n, 128).to(torch.bfloat16).cuda()
    k_pe = pe_src[:, 32:96]
    s = random_slots(n, S, 5, pad=(100,))
    run_and_compare(gpu, kv_a, torch.from_numpy(s).cuda(), random_cache((S, 576), 6), 0.5, x2=k_pe)


def test_unaligned_rows_take_the_element_path(gpu):
    """dim 100 / dim2 4 (not multiples of 8), three heads, odd strides."""
    torch.manual_seed(3)
    n, pages, page = 50, 4, 16
    src = torch.randn(n, 3 * 101).to(torch.bfloat16).cuda()
    x = src[:, :303].view(n, 3, 101)[:, :, :100]
    x2 = torch.randn(n, 3, 4).to(torch.bfloat16).cuda()
    s = random_slots(n, pages * page, 7)
    run_and_compare(gpu, x, torch.from_numpy(s).cuda(), random_cache((pages, 3, page, 104), 8), 1.75, x2=x2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("scale", [None, 0.1234567])
def test_every_bit_pattern(gpu, dtype, scale):
    """All 65536 16-bit patterns (NaN, inf, subnormals, saturation) through the store."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.int16)
    x = torch.from_numpy(bits).view(dtype).reshape(512, 1, 128).cuda()
    s = random_slots(512, 4 * 128, 9)
    run_and_compare(gpu, x, torch.from_numpy(s).cuda(), random_cache((4, 1, 128, 128), 10), scale)


def test_empty_call_is_a_noop(gpu):
    cache = random_cache((2, 128, 128), 11)
    before = cache.clone()
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    gpu.fp8_cache_store(x, torch.empty(0, dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    assert torch.equal(cache, before)


def test_full_size_32k_prefill_store(gpu):
    """K, V and index-K of a 32768-token prompt into caches of 256 permuted pages."""
    rng = np.random.default_rng(1003)
    n, pages = 32768, 256
    table = rng.permutation(pages)
    t = np.arange(n)
    slots = torch.from_numpy((table[t // 128] * 128 + t % 128).astype(np.int64)).cuda()
    for i, (heads, scale) in enumerate([(2, 0.61), (2, 3.3), (1, 1.9)]):
        x = torch.from_numpy(rng.standard_normal((n, heads, 128), dtype=np.float32)).to(torch.bfloat16).cuda()
        shape = (pages, heads, 128, 128) if heads > 1 else (pages, 128, 128)
        run_and_compare(gpu, x if heads > 1 else x[:, 0], slots, random_cache(shape, 20 + i), scale)
