"""sparse_attn_fwd on the GPU vs the float64 oracle.

Outputs: max|out - ref| <= 2e-2 * max|ref| per tensor, |lse - ref| <= 1e-3,
max_logits within 1e-3 * max(1, |ref|); -inf must match -inf.  Bitwise
checks cover the closed forms the method fixes exactly on the GPU too.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import e4m3
from oracle import indexer as OI
from oracle import quantize as OQ
import workloads as W
from helpers import assert_attention_close, bf16_dev, dev, exact_workload_ids, host, workload

pytestmark = pytest.mark.gpu
PAGE = 128
TAB = e4m3.decode_table()


def rand_codes(rng, shape, std=1.0):
    return W.e4m3_codes((rng.standard_normal(shape) * std).astype(np.float32))


# ------------------------------------------------------------------ token mode
def token_case(T, Hq, S, topk, seed, sink=True, with_invalid=False):
    rng = np.random.default_rng(seed)
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    kv8 = rand_codes(rng, (S, 576))
    idx = np.stack([rng.choice(S, topk, replace=False) for _ in range(T)]).astype(np.int32)
    if with_invalid:
        idx[0, :] = -1                      # a query with no valid key
        idx[1, ::3] = -1
        idx[2, 5] = S + 7                   # out of range: absent
    sk = (rng.standard_normal(Hq) * 3).astype(np.float32) if sink else None
    return q8, kv8, idx, sk


def run_token(gpu, q8, kv8, idx, sm, **kw):
    sink = kw.pop("attn_sink", None)
    tl = kw.pop("topk_length", None)
    return gpu.sparse_attn_fwd(dev(q8), dev(kv8), dev(idx), sm_scale=sm, mode="token", d_v=512,
                               attn_sink=None if sink is None else dev(sink),
                               topk_length=None if tl is None else dev(tl), **kw)


def test_token_mode_tiny_mla_workload(gpu):
    wl = workload(1)
    q8 = OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale)
    got = run_token(gpu, q8, wl.kv8, wl.indices, wl.sm_scale, q_scale=wl.q_scale, k_scale=wl.k_scale,
                    v_scale=wl.v_scale, attn_sink=wl.sink)
    ref = OA.sparse_attn_token(q8, wl.kv8, wl.indices, sm_scale=wl.sm_scale, d_v=512, q_scale=wl.q_scale,
                               k_scale=wl.k_scale, v_scale=wl.v_scale, attn_sink=wl.sink)
    assert_attention_close(got, ref, "mla tiny")


@pytest.mark.parametrize("Hq", [16, 128])
def test_token_mode_ragged_and_invalid(gpu, Hq):
    q8, kv8, idx, sk = token_case(6, Hq, 3000, 300, seed=Hq, with_invalid=True)
    got = run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=0.7, k_scale=1.3, v_scale=0.9, attn_sink=sk)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, q_scale=0.7, k_scale=1.3, v_scale=0.9,
                               attn_sink=sk)
    assert_attention_close(got, ref, f"token Hq={Hq}")


@pytest.mark.parametrize("Hq", [16, 128])
def test_token_mode_topk_length_and_no_sink(gpu, Hq):
    q8, kv8, idx, _ = token_case(5, Hq, 2000, 200, seed=3, sink=False)
    tl = np.array([200, 1, 0, 77, 130], np.int32)
    got = run_token(gpu, q8, kv8, idx, 1 / 24, topk_length=tl)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, topk_length=tl)
    assert_attention_close(got, ref, "topk_length")
    out, ml, lse = (host(x) for x in got)
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2])) and np.all(np.isneginf(ml[2]))


@pytest.mark.parametrize("Hq", [16, 128])
def test_token_mode_separate_v(gpu, Hq):
    q8, kv8, idx, sk = token_case(4, Hq, 1000, 96, seed=4)
    v8 = rand_codes(np.random.default_rng(5), (1000, 512))
    got = gpu.sparse_attn_fwd(dev(q8), dev(kv8), dev(idx), sm_scale=1 / 24, mode="token", v=dev(v8),
                              attn_sink=dev(sk))
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, v8=v8, attn_sink=sk)
    assert_attention_close(got, ref, "separate v")


def test_token_mode_long_mla_sampled(gpu):
    """Full-size long MLA prefill: 4096 x 128 heads, top-2048 of 65536, sink."""
    wl = workload(4)
    q8 = OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale)
    got = run_token(gpu, q8, wl.kv8, wl.indices, wl.sm_scale, attn_sink=wl.sink)
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(q8.shape[0], 12, replace=False))
    ref = OA.sparse_attn_token(q8, wl.kv8, wl.indices, sm_scale=wl.sm_scale, d_v=512, attn_sink=wl.sink,
                               tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "long mla sampled")


@pytest.mark.parametrize("T,Hq,topk", [(3, 128, 2048), (2, 256, 1000)])
def test_token_mode_split_lists(gpu, T, Hq, topk):
    """Few tokens: the key lists are split over workgroups and merged."""
    q8, kv8, idx, sk = token_case(T, Hq, 9000, topk, seed=T + Hq, with_invalid=False)
    idx[0, 100:140] = -1                    # a ragged run of absent keys inside one split
    tl = np.array([topk, topk - 45, 33][:T], np.int32)
    got = run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=0.9, attn_sink=sk, topk_length=tl)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, q_scale=0.9, attn_sink=sk,
                               topk_length=tl)
    assert_attention_close(got, ref, f"split lists T={T} Hq={Hq}")


def test_token_mode_first_tiles_absent(gpu):
    """The first key tiles hold no valid id: the reference maximum starts later."""
    q8, kv8, idx, sk = token_case(4, 128, 3000, 200, seed=21)
    idx[:, :70] = -1
    idx[1, :] = -1
    idx[1, 199] = 42                        # a single key in the last, ragged tile
    got = run_token(gpu, q8, kv8, idx, 1 / 24, attn_sink=sk)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, attn_sink=sk)
    assert_attention_close(got, ref, "first tiles absent")


def test_token_mode_late_large_logits(gpu):
    """A key far above the first tile's maximum forces the exact-maximum rerun.

    The large logits come from single exact products (rows that are zero but
    for dimension 0), so they carry no accumulation error."""
    rng = np.random.default_rng(31)
    T, Hq, S, topk = 3, 128, 2000, 160
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    q8[:, :, 0] = W.e4m3_codes(rng.uniform(32, 64, (T, Hq)).astype(np.float32))
    kv8 = rand_codes(rng, (S, 576), 0.02)
    kv8[:, 0] = 0
    # first tiles from rows < 1000, the rest from rows >= 1000
    idx = np.stack([np.concatenate([rng.choice(1000, 32, replace=False), 1000 + rng.choice(1000, topk - 32, replace=False)])
                    for _ in range(T)]).astype(np.int32)
    for t in range(T):
        for j in (90 + t, 150):             # two large keys, tiles 2 and 4
            kv8[idx[t, j]] = 0
            kv8[idx[t, j], 0] = W.e4m3_codes(rng.uniform(256, 448, 1).astype(np.float32))[0]
    got = run_token(gpu, q8, kv8, idx, 1 / 24)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512)
    # the first tile's logits are tiny; the large ones sit past the headroom above them
    z0 = np.einsum("thd,tkd->thk", TAB[q8].astype(np.float64), TAB[kv8[idx[:, :32]]].astype(np.float64)) / 24
    assert np.abs(z0).max() < 1 and ref[1].min() > 64 * math.log(2) + 1
    assert_attention_close(got, ref, "late large logits (token)")


# 128-head groups with at least 256 tokens keep each key list whole (one
# workgroup per token and head group, final outputs written directly); the
# smaller cases above split the lists and merge the partial results
def test_token_mode_unsplit_lists_edge_cases(gpu):
    q8, kv8, idx, sk = token_case(260, 128, 3000, 96, seed=41, with_invalid=True)
    idx[3:9, :40] = -1                       # first tiles absent
    idx[9, :] = -1
    idx[9, 95] = 7                           # one key, in the last tile
    tl = np.full(260, 96, np.int32)
    tl[10], tl[11], tl[12], tl[13] = 0, 1, 31, 33
    v8 = rand_codes(np.random.default_rng(42), (3000, 512))
    got = gpu.sparse_attn_fwd(dev(q8), dev(kv8), dev(idx), sm_scale=1 / 24, mode="token", v=dev(v8),
                              q_scale=0.8, k_scale=1.1, v_scale=0.6, attn_sink=dev(sk), topk_length=dev(tl))
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, v8=v8, q_scale=0.8, k_scale=1.1,
                               v_scale=0.6, attn_sink=sk, topk_length=tl)
    assert_attention_close(got, ref, "unsplit lists, edge cases")
    out, ml, lse = (host(x) for x in got)
    assert np.all(out[10] == 0) and np.all(np.isneginf(ml[10]))     # empty list: sink only


def test_token_mode_unsplit_lists_late_large_logits(gpu):
    """The exact-maximum rerun on the unsplit-list path (large logits from single exact products)."""
    rng = np.random.default_rng(43)
    T, Hq, S, topk = 256, 128, 2000, 96
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    q8[:, :, 0] = W.e4m3_codes(rng.uniform(32, 64, (T, Hq)).astype(np.float32))
    kv8 = rand_codes(rng, (S, 576), 0.02)
    kv8[:, 0] = 0
    idx = np.stack([np.concatenate([rng.choice(1000, 32, replace=False), 1000 + rng.choice(1000, topk - 32, replace=False)])
                    for _ in range(T)]).astype(np.int32)
    big = rng.choice(np.arange(1000, 2000), 40, replace=False)
    kv8[big] = 0
    kv8[big, 0] = W.e4m3_codes(rng.uniform(256, 448, 40).astype(np.float32))
    got = run_token(gpu, q8, kv8, idx, 1 / 24)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512)
    assert ref[1].max() > 64 * math.log(2) + 1
    assert_attention_close(got, ref, "late large logits (unsplit lists)")


def test_token_mode_unsplit_lists_single_key_bitwise(gpu):
    q8, kv8, _, _ = token_case(256, 128, 500, 64, seed=44, sink=False)
    idx = np.full((256, 64), -1, np.int32)
    idx[:, 37] = np.arange(256) % 500
    out, ml, lse = (host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, v_scale=2.0))
    want = 2.0 * TAB[kv8[idx[:, 37], :512]].astype(np.float64)
    assert np.array_equal(out, np.broadcast_to(want[:, None, :], out.shape))


# ------------------------------------------------------------------ GPU closed forms
@pytest.mark.parametrize("Hq", [16, 128])
def test_single_key_gives_v_bitwise(gpu, Hq):
    q8, kv8, _, _ = token_case(3, Hq, 500, 4, seed=7, sink=False)
    idx = np.full((3, 4), -1, np.int32)
    idx[:, 0] = [5, 17, 499]
    out, ml, lse = (host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, v_scale=2.0))
    for t, j in enumerate([5, 17, 499]):
        v = TAB[kv8[j, :512]] * 2.0
        expect = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().numpy()
        assert np.array_equal(out[t], np.broadcast_to(expect, out[t].shape))
        # lse = max_logits = z_j, up to the e4m3 MFMA's accumulation of the
        # 576-term dot (about 16 bits relative to its largest addend): the
        # lse tolerance of the op
        z = (TAB[q8[t]] @ TAB[kv8[j]]) / 24
        assert np.allclose(lse[t], z, rtol=0, atol=1e-3) and np.allclose(ml[t], z, rtol=0, atol=1e-3)


@pytest.mark.parametrize("pos", [0, 70, 130, 255])
def test_latent_rows_single_key_in_any_tile_half_bitwise(gpu, pos):
    # 128 q heads, V = the leading 512 bytes of each K row: the kernel scores
    # 64-key halves of 128-key tiles, each half with its own P exponent, and
    # splits P into two e4m3 codes; one valid entry in either half of the
    # first or a later tile still gives V exactly
    q8, kv8, _, _ = token_case(2, 128, 600, 4, seed=21, sink=False)
    idx = np.full((2, 256), -1, np.int32)
    idx[0, pos], idx[1, pos] = 11, 599
    out, ml, lse = (host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, v_scale=0.5))
    for t, j in enumerate([11, 599]):
        v = TAB[kv8[j, :512]] * 0.5
        expect = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().numpy()
        assert np.array_equal(out[t], np.broadcast_to(expect, out[t].shape))
        z = (TAB[q8[t]] @ TAB[kv8[j]]) / 24
        assert np.allclose(lse[t], z, rtol=0, atol=1e-3) and np.allclose(ml[t], z, rtol=0, atol=1e-3)


def test_latent_rows_and_separate_v_match_the_oracle(gpu):
    # the same inputs through the latent-row kernel (no V argument) and the
    # separate-V kernel; 1000 entries leave a last tile of 64 + 40 keys
    q8, kv8, idx, sk = token_case(6, 128, 4096, 1000, seed=22)
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, attn_sink=sk)
    a = run_token(gpu, q8, kv8, idx, 1 / 24, attn_sink=sk)
    b = gpu.sparse_attn_fwd(dev(q8), dev(kv8), dev(idx), sm_scale=1 / 24, mode="token",
                            v=dev(kv8[:, :512].copy()), attn_sink=dev(sk))
    assert_attention_close(a, ref, "latent rows")
    assert_attention_close(b, ref, "separate v")


@pytest.mark.parametrize("Hq", [16, 128])
def test_scale_invariants_bitwise(gpu, Hq):
    q8, kv8, idx, sk = token_case(4, Hq, 2000, 130, seed=8)
    base = [host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=0.75, k_scale=1.5, v_scale=1.25,
                                       attn_sink=sk)]
    # (q, k, sink) -> (2q, k/2, sink/2): identical bits
    b2 = [host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=1.5, k_scale=0.75, v_scale=1.25,
                                     attn_sink=sk / 2)]
    for x, y in zip(base, b2):
        assert np.array_equal(x, y)
    # v_scale doubles out bitwise, leaves lse and max_logits
    b3 = [host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=0.75, k_scale=1.5, v_scale=2.5,
                                     attn_sink=sk)]
    assert np.array_equal(2 * base[0], b3[0])
    assert np.array_equal(base[1], b3[1]) and np.array_equal(base[2], b3[2])
    # None == 1.0 bitwise
    n1 = [host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24)]
    n2 = [host(x) for x in run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=1.0, k_scale=1.0, v_scale=1.0)]
    for x, y in zip(n1, n2):
        assert np.array_equal(x, y)


def test_k_scale_never_touches_sink_bitwise(gpu):
    q8, kv8, idx, sk = token_case(3, 16, 1000, 64, seed=9)
    zk = np.zeros_like(kv8)
    v8 = kv8[:, :512].copy()
    a = [host(x) for x in gpu.sparse_attn_fwd(dev(q8), dev(zk), dev(idx), sm_scale=1 / 24, mode="token",
                                              v=dev(v8), k_scale=0.5, attn_sink=dev(sk))]
    b = [host(x) for x in gpu.sparse_attn_fwd(dev(q8), dev(zk), dev(idx), sm_scale=1 / 24, mode="token",
                                              v=dev(v8), k_scale=7.0, attn_sink=dev(sk))]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("Hq", [16, 128])
def test_sink_only_gives_zero(gpu, Hq):
    q8, kv8, idx, _ = token_case(2, Hq, 100, 8, seed=10, sink=False)
    idx[:] = -1
    sink = np.linspace(-3, 3, Hq).astype(np.float32)
    out, ml, lse = (host(x) for x in run_token(gpu, q8, kv8, idx, 0.5, q_scale=2.0, attn_sink=sink))
    assert np.all(out == 0)
    assert np.allclose(lse, np.broadcast_to(sink * 1.0, lse.shape), atol=1e-6)
    assert np.all(np.isneginf(ml))


# ------------------------------------------------------------------ block mode
def block_case(seq_lens, q_lens, seed, topk, Hq=16, Hkv=2, Hidx=4, scales=None, sink=False):
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    nbs = [(s + PAGE - 1) // PAGE for s in seq_lens]
    max_blocks = max(nbs)
    P = sum(nbs) + 2
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((B, max_blocks), -1, np.int32)
    o = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[o:o + nb]
        o += nb
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    q8 = rand_codes(rng, (T, Hq, 128), 1.5)
    kc = rand_codes(rng, (P, Hkv, PAGE, 128))
    vc = rand_codes(rng, (P, Hkv, PAGE, 128))
    iq = rand_codes(rng, (T, Hidx, 128))
    ik = rand_codes(rng, (P, PAGE, 128))
    sl = np.asarray(seq_lens, np.int32)
    ids = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.1, topk=topk)     # oracle ids as the input
    sk = (rng.standard_normal(Hq) * 4).astype(np.float32) if sink else None
    return dict(q8=q8, kc=kc, vc=vc, ids=ids, bt=bt, cu=cu, sl=sl, mq=max(q_lens), sink=sk)


def run_block(gpu, c, sm=0.088, **kw):
    return gpu.sparse_attn_fwd(dev(c["q8"]), dev(c["kc"]), dev(c["ids"]), v=dev(c["vc"]), sm_scale=sm,
                               mode="block", block_table=dev(c["bt"]), cu_seqlens_q=dev(c["cu"]),
                               seq_lens=dev(c["sl"]), max_q_len=c["mq"],
                               attn_sink=None if c["sink"] is None else dev(c["sink"]), **kw)


def ref_block(c, sm=0.088, tokens=None, **kw):
    return OA.sparse_attn_block(c["q8"], c["kc"], c["vc"], c["ids"], c["bt"], c["cu"], c["sl"], sm_scale=sm,
                                attn_sink=c["sink"], tokens=tokens, **kw)


@pytest.mark.parametrize("topk", [4, 64])
def test_block_prefill_several_tiles(gpu, topk):
    c = block_case([2000], [2000], seed=topk, topk=topk)
    got = run_block(gpu, c, q_scale=0.8, k_scale=1.25, v_scale=0.5)
    toks = np.arange(0, 2000, 3)
    ref = ref_block(c, tokens=toks, q_scale=0.8, k_scale=1.25, v_scale=0.5)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, f"block prefill k={topk}")


def test_block_varlen_prefix_decode_mix_with_sink(gpu):
    c = block_case([1700, 900, 5000, 129, 1], [600, 900, 1, 1, 1], seed=11, topk=6, sink=True)
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, "varlen")


def test_block_short_prefill_converts_in_kernel(gpu):
    """Fewer than 4 query tiles per sequence: V is converted inside the tile
    loop instead of by the V^T pre-pass (the long cases above use the pre-pass)."""
    c = block_case([3000, 2100], [80, 70], seed=17, topk=8, sink=True)
    got = run_block(gpu, c, q_scale=1.1, v_scale=0.7)
    ref = ref_block(c, q_scale=1.1, v_scale=0.7)
    assert_attention_close(got, ref, "short prefill")


def test_block_decode_batch(gpu):
    rng = np.random.default_rng(12)
    seq = [int(x) for x in rng.integers(1, 12000, 14)] + [1, 128, 129]
    c = block_case(seq, [1] * len(seq), seed=13, topk=16)
    got = run_block(gpu, c, v_scale=3.0)
    ref = ref_block(c, v_scale=3.0)
    assert_attention_close(got, ref, "decode")


def test_block_head_layouts(gpu):
    # 8 q heads, 8 kv heads (G = 1), 2 index heads (4 q heads each)
    c = block_case([700], [700], seed=14, topk=3, Hq=8, Hkv=8, Hidx=2)
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, "G=1")
    # 32 q heads over 1 kv head, 8 index heads
    c = block_case([900, 300], [900, 50], seed=15, topk=2, Hq=32, Hkv=1, Hidx=8)
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, "G=32")


def test_block_rows_with_no_blocks(gpu):
    c = block_case([600], [600], seed=16, topk=4)
    c["ids"] = c["ids"].copy()
    c["ids"][:, 100:110] = -1           # rows that selected nothing
    c["ids"][1, 300:305, 0] = 99        # id beyond the table: absent
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, "empty rows")
    out, ml, lse = (host(x) for x in got)
    assert np.all(out[100:110] == 0) and np.all(np.isneginf(lse[100:110]))


@pytest.mark.parametrize("topk", [7, 8])
def test_block_prefill_late_large_logits(gpu, topk):
    """Rows whose first blocks carry tiny logits and a later block logits far
    above them (beyond what fp32 can hold relative to the first reference):
    the kernel must rescan with the exact row maxima.  The late block's keys
    have one non-zero coordinate, so its dots are single exact products: the
    fp8 MFMA accumulates with ~16 bits relative to the largest addend, which
    would otherwise blur logits in the hundreds by more than the lse bound.
    top-7 leaves the last rows with more causal blocks than they select (the
    16-row-wave kernel); top-8 covers every row's blocks (the 32-row-wave
    kernel)."""
    c = block_case([900], [900], seed=17, topk=topk)
    rng = np.random.default_rng(17)
    kc = c["kc"].copy()
    bt = c["bt"][0]
    kc[bt[:3]] = rand_codes(rng, (3,) + kc.shape[1:], 0.02)
    kc[bt[4]] = 0
    kc[bt[4], :, :, 0] = W.e4m3_codes(rng.uniform(256, 448, kc.shape[1:3]).astype(np.float32))
    c["kc"] = kc
    nb = np.arange(900) // PAGE + 1
    ids = np.where(np.arange(topk)[None, :] < nb[:, None], np.arange(topk)[None, :], -1).astype(np.int32)
    c["ids"] = np.broadcast_to(ids[None], (4, 900, topk)).copy()
    got = run_block(gpu, c)
    ref = ref_block(c)
    ml = ref[2]
    assert ml[PAGE * 4:].max() - ml[:PAGE * 3].max() > 64 * math.log(2)   # the case is really exercised
    assert_attention_close(got, ref, "late large logits")


def test_block_prefill_8k_full_size_sampled(gpu):
    """8k causal prefill at full size: every row selects all of its causal
    blocks (the closed-form ids), so the attention is dense causal."""
    wl = workload(2)
    q8 = OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale)
    T = q8.shape[0]
    nb = np.arange(T) // PAGE + 1
    ids = np.where(np.arange(wl.topk)[None, :] < nb[:, None], np.arange(wl.topk)[None, :], -1)
    ids = np.ascontiguousarray(np.broadcast_to(ids[None], (4, T, wl.topk)).astype(np.int32))
    toks = np.unique(np.concatenate([np.random.default_rng(2).choice(T, 40, replace=False),
                                     [0, 1, 31, 32, 127, 128, T - 1]]))
    got = gpu.sparse_attn_fwd(dev(q8), dev(wl.k_cache8), dev(ids), v=dev(wl.v_cache8), sm_scale=wl.sm_scale,
                              mode="block", block_table=dev(wl.block_table), cu_seqlens_q=dev(wl.cu_seqlens_q),
                              seq_lens=dev(wl.seq_lens), max_q_len=wl.max_q_len, q_scale=wl.q_scale,
                              k_scale=wl.k_scale, v_scale=wl.v_scale)
    ref = OA.sparse_attn_block(q8, wl.k_cache8, wl.v_cache8, ids, wl.block_table, wl.cu_seqlens_q, wl.seq_lens,
                               sm_scale=wl.sm_scale, q_scale=wl.q_scale, k_scale=wl.k_scale,
                               v_scale=wl.v_scale, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "workload 2")


def test_block_prefill_32k_full_size_oracle_ids(gpu):
    """32k causal prefill at full size with U(0.1, 4) scales, on the oracle's
    complete id tensor for the exact-mode index codes (every row's own top-64,
    so every query tile walks the block unions the bench meets).  96 rows
    compared, spread over tile positions: the first, last and middle rows of
    32-token tiles, rows at 128-token block edges, and random rows."""
    wl = workload(3)
    _, _, ids = exact_workload_ids(3)
    q8 = OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale)
    T = q8.shape[0]
    rng = np.random.default_rng(3)
    tiles = rng.choice(T // 32, 24, replace=False) * 32
    toks = np.unique(np.concatenate([tiles, tiles + 31, tiles + 15, [0, 127, 128, 8191, 8192, 8319, T - 1],
                                     rng.choice(T, 40, replace=False)]))
    assert len(toks) >= 64
    got = gpu.sparse_attn_fwd(dev(q8), dev(wl.k_cache8), dev(ids), v=dev(wl.v_cache8), sm_scale=wl.sm_scale,
                              mode="block", block_table=dev(wl.block_table), cu_seqlens_q=dev(wl.cu_seqlens_q),
                              seq_lens=dev(wl.seq_lens), max_q_len=wl.max_q_len, q_scale=wl.q_scale,
                              k_scale=wl.k_scale, v_scale=wl.v_scale)
    ref = OA.sparse_attn_block(q8, wl.k_cache8, wl.v_cache8, ids, wl.block_table, wl.cu_seqlens_q, wl.seq_lens,
                               sm_scale=wl.sm_scale, q_scale=wl.q_scale, k_scale=wl.k_scale,
                               v_scale=wl.v_scale, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "workload 3")


def test_block_decode_full_size_oracle_ids(gpu):
    """Decode: 64 sequences x 32k tokens, every sequence on the oracle's top-64
    blocks of the exact-mode index codes, all 64 x 16 rows compared."""
    wl = workload(5)
    _, _, ids = exact_workload_ids(5)
    q8 = OQ.quantize(wl.q_bf16, OQ.BF16, wl.q_scale)
    got = gpu.sparse_attn_fwd(dev(q8), dev(wl.k_cache8), dev(ids), v=dev(wl.v_cache8), sm_scale=wl.sm_scale,
                              mode="block", block_table=dev(wl.block_table), cu_seqlens_q=dev(wl.cu_seqlens_q),
                              seq_lens=dev(wl.seq_lens), max_q_len=1)
    ref = OA.sparse_attn_block(q8, wl.k_cache8, wl.v_cache8, ids, wl.block_table, wl.cu_seqlens_q, wl.seq_lens,
                               sm_scale=wl.sm_scale)
    assert_attention_close(got, ref, "decode full")


# Decode tiles of at most 16 rows (q heads per kv head x query tokens) run the
# streamed decode kernel, each wave walking its own share of the block union.
@pytest.mark.parametrize("Hq,Hkv,Hidx,q_len", [(16, 2, 4, 1), (32, 2, 4, 1), (8, 8, 2, 1), (4, 2, 2, 1),
                                               (16, 2, 4, 2), (8, 2, 2, 4), (16, 1, 16, 1)])
def test_block_decode_streamed_head_layouts(gpu, Hq, Hkv, Hidx, q_len):
    rng = np.random.default_rng(Hq * 100 + Hkv * 10 + q_len)
    seq = [int(x) for x in rng.integers(q_len, 9000, 9)] + [q_len, 128, 129, 8192]
    c = block_case(seq, [q_len] * len(seq), seed=Hq + Hidx + q_len, topk=24, Hq=Hq, Hkv=Hkv, Hidx=Hidx,
                   sink=True)
    got = run_block(gpu, c, q_scale=0.9, k_scale=1.1, v_scale=2.0)
    ref = ref_block(c, q_scale=0.9, k_scale=1.1, v_scale=2.0)
    assert_attention_close(got, ref, f"decode Hq={Hq} Hkv={Hkv} Hidx={Hidx} q_len={q_len}")


@pytest.mark.parametrize("topk", [1, 2, 31, 32, 33, 48, 64])
def test_block_decode_streamed_split_edges(gpu, topk):
    """Lists just below, at and above one split's worth of blocks (and a
    single-block list), over sequences both shorter and longer than k blocks."""
    seq = [1, 100, 4000, 9000, 16000, 30000]
    c = block_case(seq, [1] * len(seq), seed=topk, topk=topk)
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, f"decode k={topk}")


def test_block_decode_streamed_empty_rows_and_absent_ids(gpu):
    seq = [5000, 3000, 700, 12000]
    c = block_case(seq, [1] * 4, seed=41, topk=16, sink=True)
    c["ids"] = c["ids"].copy()
    c["ids"][:, 1] = -1                 # a sequence that selected nothing
    c["ids"][2, 3, :5] = 1000           # ids beyond the table: absent
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, "decode empty rows")
    out, ml, lse = (host(x) for x in got)
    assert np.all(out[1] == 0) and np.all(np.isneginf(ml[1]))


def test_block_decode_streamed_late_large_logits(gpu):
    """Decode rows whose first selected blocks carry tiny logits and a later
    block logits beyond fp32's range relative to them: each wave reruns its
    share with the exact maxima (single exact products in the large block,
    as in the prefill case above)."""
    seq = [1500, 2000]
    c = block_case(seq, [1, 1], seed=43, topk=12)
    rng = np.random.default_rng(43)
    kc = c["kc"].copy()
    for b in range(2):
        bt = c["bt"][b]
        kc[bt[:8]] = rand_codes(rng, (8,) + kc.shape[1:], 0.02)
        kc[bt[10]] = 0
        kc[bt[10], :, :, 0] = W.e4m3_codes(rng.uniform(256, 448, kc.shape[1:3]).astype(np.float32))
    c["kc"] = kc
    ids = np.full((4, 2, 12), -1, np.int32)
    ids[:, 0, :12] = np.arange(12)
    ids[:, 1, :12] = np.arange(12)
    c["ids"] = ids
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert ref[2].max() > 64 * math.log(2) + 5    # far beyond the tiny blocks that start each share
    assert_attention_close(got, ref, "decode late large logits")


# Decode tiles of more than 16 rows (q heads per kv head x query tokens of a
# sequence, at most 64) run the tile kernel with 4 waves x 16 rows; the block
# union is split over workgroups and the partials merged by the combine kernel.
@pytest.mark.parametrize("Hq,Hkv,Hidx,q_len", [(16, 2, 4, 3), (16, 2, 4, 4), (16, 2, 4, 8), (32, 1, 8, 1),
                                               (64, 1, 16, 1), (12, 4, 4, 1)])
def test_block_decode_tile_head_layouts(gpu, Hq, Hkv, Hidx, q_len):
    rng = np.random.default_rng(Hq * 1000 + Hkv * 10 + q_len)
    seq = [int(x) for x in rng.integers(q_len, 9000, 7)] + [q_len, 128 + q_len, 8192]
    c = block_case(seq, [q_len] * len(seq), seed=Hq + Hkv + q_len, topk=24, Hq=Hq, Hkv=Hkv, Hidx=Hidx, sink=True)
    c["ids"] = c["ids"].copy()
    c["ids"][:, q_len:2 * q_len] = -1           # a sequence whose rows selected nothing
    c["ids"][0, 0, :3] = 5000                   # ids beyond the table: absent
    got = run_block(gpu, c, q_scale=0.9, k_scale=1.1, v_scale=2.0)
    ref = ref_block(c, q_scale=0.9, k_scale=1.1, v_scale=2.0)
    assert_attention_close(got, ref, f"tile decode Hq={Hq} Hkv={Hkv} Hidx={Hidx} q_len={q_len}")
    out, ml, lse = (host(x) for x in got)
    assert np.all(out[q_len:2 * q_len] == 0) and np.all(np.isneginf(ml[q_len:2 * q_len]))
    assert np.all(np.isfinite(lse[q_len:2 * q_len]))      # the sink alone


@pytest.mark.parametrize("topk", [1, 7, 8, 9, 16, 17, 33, 64])
def test_block_decode_tile_split_edges(gpu, topk):
    """Multi-token decode (4 queries x 8 q heads per kv head = 32 rows): union
    sizes just below, at and above one workgroup's 32 blocks."""
    seq = [4, 100, 4000, 9000, 16000, 30000]
    c = block_case(seq, [4] * len(seq), seed=200 + topk, topk=topk)
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert_attention_close(got, ref, f"tile decode k={topk}")


def test_block_decode_tile_late_large_logits(gpu):
    """Tile decode rows whose first blocks carry tiny logits and a later block
    logits far above them: the workgroup reruns its share with the exact maxima."""
    seq = [1500, 2000]
    c = block_case(seq, [4, 4], seed=47, topk=12)
    rng = np.random.default_rng(47)
    kc = c["kc"].copy()
    for b in range(2):
        bt = c["bt"][b]
        kc[bt[:8]] = rand_codes(rng, (8,) + kc.shape[1:], 0.02)
        kc[bt[10]] = 0
        kc[bt[10], :, :, 0] = W.e4m3_codes(rng.uniform(256, 448, kc.shape[1:3]).astype(np.float32))
    c["kc"] = kc
    c["ids"] = np.broadcast_to(np.arange(12, dtype=np.int32)[None, None], (4, 8, 12)).copy()
    got = run_block(gpu, c)
    ref = ref_block(c)
    assert ref[2].max() > 64 * math.log(2) + 5
    assert_attention_close(got, ref, "tile decode late large logits")


@pytest.mark.parametrize("q_lens", [[2500], [100], [1], [4]])
def test_block_pages_outside_the_cache_add_no_keys(gpu, q_lens):
    """Selected blocks whose table entry is -1, one past the cache or far past
    it add no keys, against the oracle: prefill with the V^T pre-pass (2500
    queries) and with in-kernel V conversion (100), streamed decode (1) and
    tile decode (4 queries x 8 heads)."""
    c = block_case([2500], q_lens, seed=50 + q_lens[0], topk=8, sink=True)
    P = c["kc"].shape[0]
    c["bt"] = c["bt"].copy()
    c["bt"][0, [1, 5, 9]] = [-1, P, 10_000_000]
    ids = c["ids"].copy()
    ids[:, :, 0] = 1                 # every row selects block 1
    ids[0, :, 1] = 5
    ids[1, :, 1] = 9
    c["ids"] = ids
    got = run_block(gpu, c, q_scale=1.2, v_scale=0.5)
    ref = ref_block(c, q_scale=1.2, v_scale=0.5)
    assert_attention_close(got, ref, f"absent pages q_len={q_lens[0]}")


def test_block_prefill_wide_block_table(gpu):
    """A 4096-column block table: the per-list bitmaps no longer fit beside two
    K/V buffers, so the prefill runs the single-buffered tile kernel."""
    c = block_case([3000, 2100], [1500, 2100], seed=60, topk=8, sink=True)
    bt = np.full((2, 4096), -1, np.int32)
    bt[:, :c["bt"].shape[1]] = c["bt"]
    c["bt"] = bt
    got = run_block(gpu, c, q_scale=0.8, k_scale=1.2, v_scale=1.5)
    toks = np.arange(0, 3600, 5)
    ref = ref_block(c, tokens=toks, q_scale=0.8, k_scale=1.2, v_scale=1.5)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "wide block table")


def test_block_prefill_128_q_heads_per_kv_head(gpu):
    """128 q heads on one kv head (8 index heads): two tokens per 256-row tile."""
    c = block_case([700], [700], seed=61, topk=3, Hq=128, Hkv=1, Hidx=8, sink=True)
    got = run_block(gpu, c)
    toks = np.arange(0, 700, 7)
    ref = ref_block(c, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "G=128")


def test_token_mode_long_lists_unpipelined(gpu):
    """Index lists longer than the pipelined 128-head kernel can stage in LDS
    (more than 15104 ids per token, 256 tokens so nothing is split): the
    gather kernel with 64-key tiles."""
    rng = np.random.default_rng(70)
    T, Hq, S, topk = 256, 128, 20000, 15360
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    kv8 = rand_codes(rng, (S, 576))
    idx = np.stack([rng.permutation(S)[:topk] for _ in range(T)]).astype(np.int32)
    idx[0, :] = -1
    idx[1, ::3] = -1
    tl = np.full(T, topk, np.int32)
    tl[2], tl[3] = 1, 8000
    sk = (rng.standard_normal(Hq) * 3).astype(np.float32)
    got = run_token(gpu, q8, kv8, idx, 1 / 24, q_scale=0.9, v_scale=1.5, attn_sink=sk, topk_length=tl)
    toks = np.array([0, 1, 2, 3, 100, 255])
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, q_scale=0.9, v_scale=1.5, attn_sink=sk,
                               topk_length=tl, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "long lists")


def test_token_mode_lists_past_the_latent_kernel_lds(gpu):
    """V taken from K, 4096 ids per token and 256 tokens (nothing split): the
    latent-row kernel's two 128-key K tiles leave LDS for 3584 ids, so the
    call takes the 128-head kernel with staged V^T tiles instead."""
    rng = np.random.default_rng(71)
    T, Hq, S, topk = 256, 128, 9000, 4096
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    kv8 = rand_codes(rng, (S, 576))
    idx = np.stack([rng.permutation(S)[:topk] for _ in range(T)]).astype(np.int32)
    idx[1, ::5] = -1
    tl = np.full(T, topk, np.int32)
    tl[2], tl[3] = 3, 3600
    sk = (rng.standard_normal(Hq) * 3).astype(np.float32)
    got = run_token(gpu, q8, kv8, idx, 1 / 24, k_scale=1.2, attn_sink=sk, topk_length=tl)
    toks = np.array([0, 1, 2, 3, 77, 255])
    ref = OA.sparse_attn_token(q8, kv8, idx, sm_scale=1 / 24, d_v=512, k_scale=1.2, attn_sink=sk,
                               topk_length=tl, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "lists past the latent kernel's LDS")


def test_token_mode_cache_past_2gb(gpu):
    """A 2.2 GB KV array (3.8M rows of 576 bytes): byte offsets outside the
    pipelined kernel's 32-bit range send 128-head groups to the gather kernel
    with 64-bit addressing (4 tokens: lists split over workgroups, merged)."""
    S, T, Hq, topk = 3_800_000, 4, 128, 1024
    g = torch.Generator(device="cuda").manual_seed(71)
    kv = torch.empty((S, 576), dtype=torch.uint8, device="cuda")
    for r0 in range(0, S, 400_000):
        r1 = min(S, r0 + 400_000)
        kv[r0:r1] = torch.randn((r1 - r0, 576), generator=g, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8)
    rng = np.random.default_rng(71)
    q8 = rand_codes(rng, (T, Hq, 576), 2.0)
    idx = np.stack([rng.choice(S, topk, replace=False) for _ in range(T)]).astype(np.int32)
    idx[:, :4] = [S - 1, S - 2, S - 3000, 3_700_123]          # rows past 2 GB
    idx[1, 500:600] = -1
    sk = (rng.standard_normal(Hq) * 3).astype(np.float32)
    got = gpu.sparse_attn_fwd(dev(q8), kv, dev(idx), sm_scale=1 / 24, mode="token", d_v=512, attn_sink=dev(sk),
                              k_scale=0.7)
    used = np.unique(idx[idx >= 0])
    rows = kv[torch.from_numpy(used.astype(np.int64)).cuda()].cpu().numpy()
    remap = np.full(idx.shape, -1, np.int64)
    remap[idx >= 0] = np.searchsorted(used, idx[idx >= 0])
    ref = OA.sparse_attn_token(q8, rows, remap.astype(np.int32), sm_scale=1 / 24, d_v=512, attn_sink=sk,
                               k_scale=0.7)
    del kv
    torch.cuda.empty_cache()
    assert_attention_close(got, ref, "2 GB cache")
