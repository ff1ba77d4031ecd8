"""The producers chained into the hot path on the GPU, against the same chain of
oracle functions: fp8 caches, quantized queries and ids bit-exact, attention
outputs within the acceptance tolerances."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from helpers import assert_attention_close, dev
from oracle import attention as OA
from oracle import cache_store as OCS
from oracle import indexer as OI
from oracle import quantize as OQ
from oracle import rope as ORO

pytestmark = pytest.mark.gpu
PAGE = 128


def bf16_bits(f) -> np.ndarray:
    """bf16 bit patterns of fp32 values (round to nearest even)."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_block_prefill_layer(gpu):
    """A 1200-token prompt: K / V / index-K stored into paged caches by slot, Q and
    the index query quantized, top-4 of 10 blocks selected, block attention."""
    rng = np.random.default_rng(77)
    S, Hq, Hkv, Hidx, D, topk = 1200, 16, 2, 4, 128, 4
    k_s, v_s, ik_s, q_s, iq_s = 0.7, 1.3, 2.0, 0.5, 0.25
    nb, P = (S + PAGE - 1) // PAGE, 12
    table = rng.permutation(P)[:nb].astype(np.int32).reshape(1, nb)
    t = np.arange(S)
    slots = (table[0, t // PAGE].astype(np.int64) * PAGE + t % PAGE)
    k_b = bf16_bits(rng.standard_normal((S, Hkv, D)))
    v_b = bf16_bits(rng.standard_normal((S, Hkv, D)))
    q_b = bf16_bits(rng.standard_normal((S, Hq, D)))
    # e4m3-exact integers (scaled) in the index tensors: exact index dots, so ids compare bit for bit
    ints = W.E4M3_EXACT_INTS
    ik_b = bf16_bits(rng.choice(ints[ints <= 16], (S, 1, D)) * rng.choice([-1.0, 1.0], (S, 1, D)) * ik_s)
    iq_b = bf16_bits(rng.choice(ints, (S, Hidx, D)) * rng.choice([-1.0, 1.0], (S, Hidx, D)) * iq_s)
    cu = np.array([0, S], np.int32)
    sl = np.array([S], np.int32)

    # GPU chain
    kc = torch.zeros((P, Hkv, PAGE, D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ikc = torch.zeros((P, PAGE, D), dtype=torch.uint8, device="cuda")
    sl_d = dev(slots)
    gpu.fp8_cache_store(bf16_tensor(k_b), sl_d, kc, scale=k_s)
    gpu.fp8_cache_store(bf16_tensor(v_b), sl_d, vc, scale=v_s)
    gpu.fp8_cache_store(bf16_tensor(ik_b[:, 0]), sl_d, ikc, scale=ik_s)
    q8 = gpu.fp8_quantize(bf16_tensor(q_b), q_s)
    iq8 = gpu.fp8_quantize(bf16_tensor(iq_b), iq_s)
    ids = gpu.indexer_topk(iq8, ikc, dev(table), dev(cu), dev(sl), max_q_len=S, sm_scale=1 / math.sqrt(D),
                           topk=topk, idx_q_scale=iq_s, idx_k_scale=ik_s)
    got = gpu.sparse_attn_fwd(q8, kc, ids, v=vc, sm_scale=1 / math.sqrt(D), mode="block", block_table=dev(table),
                              cu_seqlens_q=dev(cu), seq_lens=dev(sl), max_q_len=S, q_scale=q_s, k_scale=k_s,
                              v_scale=v_s)
    torch.cuda.synchronize()

    # oracle chain
    zeros = np.zeros((P, Hkv, PAGE, D), np.uint8)
    r_kc = OCS.cache_store(zeros, k_b, OQ.BF16, slots, k_s)
    r_vc = OCS.cache_store(zeros, v_b, OQ.BF16, slots, v_s)
    r_ikc = OCS.cache_store(np.zeros((P, 1, PAGE, D), np.uint8), ik_b, OQ.BF16, slots, ik_s)[:, 0]
    r_q8 = OQ.quantize(q_b, OQ.BF16, q_s)
    r_iq8 = OQ.quantize(iq_b, OQ.BF16, iq_s)
    r_ids = OI.indexer_topk(r_iq8, r_ikc, table, cu, sl, sm_scale=1 / math.sqrt(D), topk=topk,
                            idx_q_scale=iq_s, idx_k_scale=ik_s)
    assert np.array_equal(kc.cpu().numpy(), r_kc) and np.array_equal(vc.cpu().numpy(), r_vc)
    assert np.array_equal(ikc.cpu().numpy(), r_ikc)
    assert np.array_equal(q8.cpu().numpy(), r_q8) and np.array_equal(iq8.cpu().numpy(), r_iq8)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    toks = np.arange(0, S, 7)
    ref = OA.sparse_attn_block(r_q8, r_kc, r_vc, r_ids, table, cu, sl, sm_scale=1 / math.sqrt(D), q_scale=q_s,
                               k_scale=k_s, v_scale=v_s, tokens=toks)
    out, ml, lse = got
    assert_attention_close((out[toks], ml[toks], lse[toks]), ref, "block prefill layer")


@pytest.mark.parametrize("neox", [True, False])
def test_mla_prefill_layer(gpu, neox):
    """MLA: queries roped and quantized in one pass, latent + rotated rope key rows
    packed into the flat fp8 KV array by slot, token-sparse attention with a sink."""
    rng = np.random.default_rng(78)
    T, Hq, S, topk = 96, 16, 2000, 128
    R, pos_max = 64, 4096
    i = np.arange(R // 2)
    ang = np.arange(pos_max)[:, None] * 10000.0 ** (-2.0 * i / R)[None, :]
    cs = np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)
    q_b = bf16_bits(rng.standard_normal((T, Hq, 576)))
    pos = rng.integers(0, pos_max, T).astype(np.int64)
    kv_a = bf16_bits(rng.standard_normal((S, 512)))
    k_pe = bf16_bits(rng.standard_normal((S, 64)))           # already rotated by the model
    slots = rng.permutation(S).astype(np.int64)
    idx = np.stack([rng.choice(S, topk, replace=False) for _ in range(T)]).astype(np.int32)
    sm, q_s, kv_s = 1 / 24, 0.5, 0.8
    sink = ((np.log(topk) + rng.standard_normal(Hq)) / (sm * q_s)).astype(np.float32)

    qt = bf16_tensor(q_b)
    q8 = gpu.fp8_rope_quantize(qt[..., 512:], dev(cs), dev(pos), x_nope=qt[..., :512], is_neox=neox, scale=q_s)
    kv8 = torch.zeros((S, 576), dtype=torch.uint8, device="cuda")
    gpu.fp8_cache_store(bf16_tensor(kv_a), dev(slots), kv8, scale=kv_s, x2=bf16_tensor(k_pe))
    got = gpu.sparse_attn_fwd(q8.view(T, Hq, 576), kv8, dev(idx), sm_scale=sm, mode="token", d_v=512,
                              q_scale=q_s, k_scale=kv_s, v_scale=kv_s, attn_sink=dev(sink))
    torch.cuda.synchronize()

    r_q8 = ORO.rope_quantize(q_b[..., :512], q_b[..., 512:], OQ.BF16, cs, pos, neox, q_s)
    r_kv8 = OCS.cache_store(np.zeros((S, 1, 1, 576), np.uint8), kv_a[:, None], OQ.BF16, slots, kv_s,
                            k_pe[:, None])[:, 0, 0]
    assert np.array_equal(q8.cpu().numpy(), r_q8)
    assert np.array_equal(kv8.cpu().numpy(), r_kv8)
    ref = OA.sparse_attn_token(r_q8, r_kv8, idx, sm_scale=sm, d_v=512, q_scale=q_s, k_scale=kv_s, v_scale=kv_s,
                               attn_sink=sink)
    assert_attention_close(got, ref, "mla prefill layer")


def test_decode_step_layer(gpu):
    """A decode step: each sequence's new K / V / index-K stored at its last
    position into caches already holding the prompt, then the index query and
    Q quantized, top-8 blocks selected and attended (the new key sees itself)."""
    rng = np.random.default_rng(79)
    B, Hq, Hkv, Hidx, D, topk = 6, 16, 2, 4, 128, 8
    seq_lens = np.array([1500, 1024, 129, 2047, 900, 1921], np.int32)
    nbs = (seq_lens + PAGE - 1) // PAGE
    mb = int(nbs.max())
    P = int(nbs.sum()) + 3
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, mb), -1, np.int32)
    o = 0
    for b in range(B):
        table[b, :nbs[b]] = perm[o:o + nbs[b]]
        o += nbs[b]
    ints = W.E4M3_EXACT_INTS
    ik_s, iq_s, k_s, v_s = 0.5, 4.0, 1.7, 0.6
    # the caches already hold the prompt (all but the last position of each sequence)
    kc0 = W.e4m3_codes((rng.standard_normal((P, Hkv, PAGE, D)) / k_s).astype(np.float32))
    vc0 = W.e4m3_codes((rng.standard_normal((P, Hkv, PAGE, D)) / v_s).astype(np.float32))
    ik0 = W.e4m3_codes((rng.choice(ints[ints <= 16], (P, PAGE, D)) * rng.choice([-1.0, 1.0], (P, PAGE, D)))
                       .astype(np.float32))
    pos = (seq_lens - 1).astype(np.int64)
    slots = table[np.arange(B), pos // PAGE].astype(np.int64) * PAGE + pos % PAGE
    k_b = bf16_bits(rng.standard_normal((B, Hkv, D)))
    v_b = bf16_bits(rng.standard_normal((B, Hkv, D)))
    ik_b = bf16_bits(rng.choice(ints[ints <= 16], (B, 1, D)) * rng.choice([-1.0, 1.0], (B, 1, D)) * ik_s)
    q_b = bf16_bits(rng.standard_normal((B, Hq, D)))
    iq_b = bf16_bits(rng.choice(ints, (B, Hidx, D)) * rng.choice([-1.0, 1.0], (B, Hidx, D)) * iq_s)
    cu = np.arange(B + 1, dtype=np.int32)

    kc, vc, ikc = dev(kc0), dev(vc0), dev(ik0)
    sl_d = dev(slots)
    gpu.fp8_cache_store(bf16_tensor(k_b), sl_d, kc, scale=k_s)
    gpu.fp8_cache_store(bf16_tensor(v_b), sl_d, vc, scale=v_s)
    gpu.fp8_cache_store(bf16_tensor(ik_b[:, 0]), sl_d, ikc, scale=ik_s)
    q8 = gpu.fp8_quantize(bf16_tensor(q_b), None)
    iq8 = gpu.fp8_quantize(bf16_tensor(iq_b), iq_s)
    ids = gpu.indexer_topk(iq8, ikc, dev(table), dev(cu), dev(seq_lens), max_q_len=1, sm_scale=1 / math.sqrt(D),
                           topk=topk, idx_q_scale=iq_s, idx_k_scale=ik_s)
    got = gpu.sparse_attn_fwd(q8, kc, ids, v=vc, sm_scale=1 / math.sqrt(D), mode="block", block_table=dev(table),
                              cu_seqlens_q=dev(cu), seq_lens=dev(seq_lens), max_q_len=1, k_scale=k_s, v_scale=v_s)
    torch.cuda.synchronize()

    r_kc = OCS.cache_store(kc0, k_b, OQ.BF16, slots, k_s)
    r_vc = OCS.cache_store(vc0, v_b, OQ.BF16, slots, v_s)
    r_ikc = OCS.cache_store(ik0[:, None], ik_b, OQ.BF16, slots, ik_s)[:, 0]
    r_q8 = OQ.quantize(q_b, OQ.BF16, None)
    r_iq8 = OQ.quantize(iq_b, OQ.BF16, iq_s)
    r_ids = OI.indexer_topk(r_iq8, r_ikc, table, cu, seq_lens, sm_scale=1 / math.sqrt(D), topk=topk,
                            idx_q_scale=iq_s, idx_k_scale=ik_s)
    assert np.array_equal(kc.cpu().numpy(), r_kc) and np.array_equal(vc.cpu().numpy(), r_vc)
    assert np.array_equal(ikc.cpu().numpy(), r_ikc)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    ref = OA.sparse_attn_block(r_q8, r_kc, r_vc, r_ids, table, cu, seq_lens, sm_scale=1 / math.sqrt(D),
                               k_scale=k_s, v_scale=v_s)
    assert_attention_close(got, ref, "decode step layer")
