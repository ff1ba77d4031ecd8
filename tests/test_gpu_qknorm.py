"""GPU parity of fp8_qknorm_rope_quantize against the oracle: codes bit-exact.

The normaliser is decided in fp64 from the sum of squares, which is exact
(and so independent of the order of the additions) for every row below; the
rest is fp32 operation by operation on both sides.  Where the oracle writes a
NaN code (an infinity in the row) either NaN code is accepted: IEEE leaves
the sign of a NaN that arithmetic creates open.
"""

import numpy as np
import pytest
import torch

from oracle import qknorm as OQN
from oracle import quantize as OQ

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


def oracle_codes(x, w, eps, cache, pos, R, neox, scale, tokens=None):
    xx = x if x.dim() == 3 else x.unsqueeze(1)
    sel = slice(None) if tokens is None else torch.as_tensor(tokens)
    dt = OQ.BF16 if x.dtype == torch.bfloat16 else OQ.FP16
    cs = cache.numpy() if cache is not None else np.zeros((1, 2), np.float32)
    p = pos.numpy()[sel] if pos is not None else np.zeros(xx[sel].shape[0], np.int64)
    return OQN.qknorm_rope_quantize(bits_of(xx[sel]), dt, w.numpy(), eps, cs, p, R, neox, scale)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("scale", [None, 0.37])
def test_index_query_rows(gpu, neox, scale):
    """[T, 4 index heads, 128] with the last 64 dims rotated."""
    torch.manual_seed(0)
    T = 300
    x = (torch.randn(T, 4, 128) * 3).to(torch.bfloat16).cuda()
    w = torch.rand(128) * 2 - 0.5
    pos = torch.randint(0, 4096, (T,), dtype=torch.int64)
    cache = roformer_cache(4096, 64)
    got = gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-6, rope_dim=64, cos_sin_cache=cache.cuda(),
                                       positions=pos.cuda(), is_neox=neox, scale=scale)
    torch.cuda.synchronize()
    assert_codes_equal(got.cpu().numpy(), oracle_codes(x, w, 1e-6, cache, pos, 64, neox, scale))


@pytest.mark.parametrize("neox", [True, False])
def test_index_key_insert_only(gpu, neox):
    """One index-K head per token stored by slot into [pages, page, 128]; no rows returned."""
    torch.manual_seed(1)
    T, pages, page = 257, 4, 128
    x = torch.randn(T, 128).to(torch.bfloat16).cuda()
    w = torch.rand(128) + 0.5
    pos = torch.arange(T, dtype=torch.int64) * 7
    cache = roformer_cache(2048, 64)
    slots = torch.from_numpy(np.random.default_rng(1).permutation(pages * page)[:T].astype(np.int64))
    slots[[3, 100]] = -1
    slots[7] = pages * page                       # out of range: skipped
    kc = torch.full((pages, page, 128), 0x55, dtype=torch.uint8, device="cuda")
    ret = gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-5, rope_dim=64, cos_sin_cache=cache.cuda(),
                                       positions=pos.cuda(), is_neox=neox, write_out=False,
                                       slot_mapping=slots.cuda(), cache=kc)
    torch.cuda.synchronize()
    assert ret is None
    codes = oracle_codes(x, w, 1e-5, cache, pos, 64, neox, None)
    want = OQN.store_rows(np.full((pages, 1, page, 128), 0x55, np.uint8), codes, slots.numpy())[:, 0]
    assert_codes_equal(kc.cpu().numpy(), want)


def test_rows_and_store_together_with_two_heads(gpu):
    torch.manual_seed(2)
    T, H, pages, page = 90, 2, 3, 64
    x = (torch.randn(T, H, 128) * 0.01).to(torch.float16).cuda()
    w = torch.randn(128)
    pos = torch.randint(0, 512, (T,), dtype=torch.int64)
    cache = roformer_cache(512, 32)
    slots = torch.arange(T, dtype=torch.int64) * 2
    kc = torch.zeros((pages, H, page, 128), dtype=torch.uint8, device="cuda")
    out = gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-6, rope_dim=32, cos_sin_cache=cache.cuda(),
                                       positions=pos.cuda(), scale=2.5, slot_mapping=slots.cuda(), cache=kc)
    torch.cuda.synchronize()
    codes = oracle_codes(x, w, 1e-6, cache, pos, 32, True, 2.5)
    assert_codes_equal(out.cpu().numpy(), codes)
    want = OQN.store_rows(np.zeros((pages, H, page, 128), np.uint8), codes, slots.numpy())
    assert_codes_equal(kc.cpu().numpy(), want)


@pytest.mark.parametrize("D,R", [(64, 16), (512, 64), (256, 0), (136, 128), (8, 0)])
def test_head_dims_and_rope_widths(gpu, D, R):
    """Head dims from one chunk to a full wave (512), rope covering the whole
    head (136 = 8 + 128) or nothing (no cos/sin needed)."""
    torch.manual_seed(D + R)
    T, H = 70, 3
    x = (torch.randn(T, H, D) * 2).to(torch.bfloat16).cuda()
    w = torch.rand(D) * 3 - 1
    pos = torch.randint(0, 1000, (T,), dtype=torch.int64) if R else None
    cache = roformer_cache(1000, R) if R else None
    for neox in (True, False):
        got = gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-6, rope_dim=R,
                                           cos_sin_cache=cache.cuda() if R else None,
                                           positions=pos.cuda() if R else None, is_neox=neox)
        torch.cuda.synchronize()
        assert_codes_equal(got.cpu().numpy(), oracle_codes(x, w, 1e-6, cache, pos, R, neox, None))


def test_special_rows(gpu):
    """Rows of zeros (eps decides r), an infinity (NaN there, signed zeros
    elsewhere), magnitudes near the ends of the bf16 range, invalid positions."""
    T = 12
    f = np.random.default_rng(3).standard_normal((T, 1, 128)).astype(np.float32)
    f[0] = 0.0
    f[1, 0, 5] = np.inf
    f[2] *= 2.0 ** 100
    f[3] *= 2.0 ** -100
    f[4, 0, 70] = -np.inf
    x = torch.from_numpy(f).to(torch.bfloat16).cuda()
    w = torch.linspace(-2, 2, 128)
    pos = torch.arange(T, dtype=torch.int64)
    pos[[5, 6]] = torch.tensor([-3, 1 << 40])
    cache = roformer_cache(64, 64)
    got = gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-6, rope_dim=64, cos_sin_cache=cache.cuda(),
                                       positions=pos.cuda())
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert_codes_equal(g, oracle_codes(x, w, 1e-6, cache, pos, 64, True, None))
    assert np.all(g[[5, 6], :, 64:] == 0x7F)


def test_into_a_preallocated_strided_output(gpu):
    torch.manual_seed(4)
    T, H = 33, 4
    xb = torch.randn(T, H, 192).to(torch.bfloat16).cuda()
    x = xb[..., 32:160]                           # a strided view of 128 dims
    buf = torch.full((T, H, 256), 0x33, dtype=torch.uint8, device="cuda")
    out = buf[..., 64:192]
    w = torch.rand(128)
    pos = torch.randint(0, 128, (T,), dtype=torch.int64)
    cache = roformer_cache(128, 64)
    gpu.fp8_qknorm_rope_quantize(x, w.cuda(), 1e-6, rope_dim=64, cos_sin_cache=cache.cuda(), positions=pos.cuda(),
                                 out=out)
    torch.cuda.synchronize()
    assert_codes_equal(out.cpu().numpy(), oracle_codes(x, w, 1e-6, cache, pos, 64, True, None))
    b = buf.cpu().numpy()
    assert np.all(b[..., :64] == 0x33) and np.all(b[..., 192:] == 0x33)


def test_full_size_index_rows_sampled(gpu):
    """32768 tokens x 4 index heads x 128 (the 32k prompt's index query), and
    its index keys stored into 256 pages of 128; 40 tokens checked."""
    g = torch.Generator(device="cuda").manual_seed(5)
    T = 32768
    q = torch.randn((T, 4, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((T, 128), generator=g, device="cuda").to(torch.bfloat16)
    wq, wk = torch.rand(128) + 0.5, torch.rand(128) + 0.5
    pos = torch.arange(T, dtype=torch.int64)
    cache = roformer_cache(T, 64)
    slots = pos.clone()
    kc = torch.empty((256, 128, 128), dtype=torch.uint8, device="cuda")
    qo = gpu.fp8_qknorm_rope_quantize(q, wq.cuda(), 1e-6, rope_dim=64, cos_sin_cache=cache.cuda(),
                                      positions=pos.cuda(), scale=0.5)
    gpu.fp8_qknorm_rope_quantize(k, wk.cuda(), 1e-6, rope_dim=64, cos_sin_cache=cache.cuda(), positions=pos.cuda(),
                                 write_out=False, slot_mapping=slots.cuda(), cache=kc)
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(6).choice(T, 40, replace=False))
    assert_codes_equal(qo.cpu().numpy()[toks], oracle_codes(q.cpu(), wq, 1e-6, cache, pos, 64, True, 0.5, toks))
    kk = oracle_codes(k.cpu(), wk, 1e-6, cache, pos, 64, True, None, toks)[:, 0]
    kcn = kc.cpu().numpy().reshape(256 * 128, 128)
    assert_codes_equal(kcn[toks], kk)
