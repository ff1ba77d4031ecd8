"""Pins for the oracle's sparse attention (CPU only)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import e4m3
from oracle import indexer as IX
from workloads import e4m3_codes

PAGE = 128
TAB = e4m3.decode_table()


def codes(x):
    return e4m3_codes(np.asarray(x, np.float32))


def rand_codes(rng, shape):
    return codes(rng.standard_normal(shape))


# ---------------------------------------------------------------- token mode

def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(0)
    S, D, Dv, n = 64, 32, 16, 9
    row = rand_codes(rng, (1, D))
    kv = np.repeat(row, S, axis=0)
    v = rand_codes(rng, (S, Dv))
    q = rand_codes(rng, (1, 3, D))
    idx = rng.choice(S, n, replace=False)[None]
    out, lse, mx = A.sparse_attn_token(q, kv, idx, sm_scale=0.3, d_v=Dv, q_scale=0.5, k_scale=2.0,
                                       v_scale=1.5, v8=v)
    mean_v = TAB[v[idx[0]]].mean(axis=0)
    assert np.allclose(out[0], 1.5 * mean_v[None], rtol=0, atol=1e-13)
    z = 0.3 * 0.5 * 2.0 * (TAB[q[0]] @ TAB[row[0]])
    assert np.allclose(lse[0], z + math.log(n), atol=1e-12)
    assert np.allclose(mx[0], z, atol=1e-12)


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(1)
    kv = rand_codes(rng, (50, 24))
    q = np.zeros((1, 2, 24), np.uint8)
    idx = np.arange(0, 50, 5)[None]
    out, lse, mx = A.sparse_attn_token(q, kv, idx, sm_scale=1.0, d_v=8)
    assert np.allclose(out[0], TAB[kv[idx[0], :8]].mean(0)[None], atol=1e-13)
    assert np.allclose(lse[0], math.log(10), atol=1e-13)
    assert np.all(mx[0] == 0.0)


def test_single_key_gives_v_exactly():
    rng = np.random.default_rng(2)
    kv = rand_codes(rng, (20, 16))
    q = rand_codes(rng, (1, 4, 16))
    idx = np.array([[7, -1, -1, -1]])
    out, lse, mx = A.sparse_attn_token(q, kv, idx, sm_scale=0.25, d_v=8, v_scale=2.0)
    assert np.array_equal(out[0], np.broadcast_to(2.0 * TAB[kv[7, :8]], (4, 8)))
    z = 0.25 * (TAB[q[0]] @ TAB[kv[7]])
    assert np.allclose(lse[0], z, atol=1e-14) and np.allclose(mx[0], z, atol=1e-14)


def test_single_key_with_sink_is_logistic():
    rng = np.random.default_rng(3)
    kv = rand_codes(rng, (10, 16))
    q = rand_codes(rng, (1, 2, 16))
    sink = np.array([0.7, -2.0])
    out, lse, mx = A.sparse_attn_token(q, kv, np.array([[4]]), sm_scale=0.5, q_scale=3.0, d_v=16,
                                       attn_sink=sink)
    z = 0.5 * 3.0 * (TAB[q[0]] @ TAB[kv[4]])
    zs = 0.5 * 3.0 * sink
    w = 1.0 / (1.0 + np.exp(-(z - zs)))
    assert np.allclose(out[0], w[:, None] * TAB[kv[4]][None], atol=1e-13)
    assert np.allclose(lse[0], np.logaddexp(z, zs), atol=1e-13)


def test_sink_only_limit():
    rng = np.random.default_rng(4)
    kv = rand_codes(rng, (10, 16))
    q = rand_codes(rng, (2, 3, 16))
    idx = np.array([[-1, -1], [1, 2]])
    sink = np.array([1.0, 2.0, 3.0])
    out, lse, mx = A.sparse_attn_token(q, kv, idx, sm_scale=0.5, q_scale=2.0, d_v=16, attn_sink=sink)
    assert np.all(out[0] == 0.0)
    assert np.allclose(lse[0], 0.5 * 2.0 * sink)
    assert np.all(np.isneginf(mx[0]))
    # a dominating sink drives the output to 0
    out2, _, _ = A.sparse_attn_token(q, kv, idx, sm_scale=0.5, d_v=16, attn_sink=np.full(3, 200.0))
    assert np.max(np.abs(out2[1])) < 1e-30


def test_empty_without_sink():
    kv = np.zeros((4, 8), np.uint8)
    q = np.zeros((1, 2, 8), np.uint8)
    out, lse, mx = A.sparse_attn_token(q, kv, np.array([[-1, -1]]), sm_scale=1.0, d_v=8)
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(np.isneginf(mx))


def test_two_keys_logistic_weights():
    # q = e0, k rows differ only in dim 0: logit gap is known exactly
    q = codes(np.eye(1, 8)[None])
    kv = codes(np.array([[3.0] + [0] * 7, [1.0] + [0] * 7]))
    out, lse, mx = A.sparse_attn_token(q, kv, np.array([[0, 1]]), sm_scale=0.5, d_v=8)
    w0 = 1.0 / (1.0 + math.exp(-(1.5 - 0.5)))
    expect = w0 * TAB[kv[0]] + (1 - w0) * TAB[kv[1]]
    assert np.allclose(out[0, 0], expect, atol=1e-14)


def _tok_case(seed=5):
    rng = np.random.default_rng(seed)
    S, Dqk, Dv, T, H, k = 300, 48, 32, 5, 4, 40
    kv = rand_codes(rng, (S, Dqk))
    q = rand_codes(rng, (T, H, Dqk))
    idx = np.stack([np.sort(rng.choice(S, k, replace=False)) for _ in range(T)])
    sink = rng.standard_normal(H) * 3
    return q, kv, idx, sink, Dv


def test_k_scale_never_touches_sink():
    q, kv, idx, sink, Dv = _tok_case()
    a = A.sparse_attn_token(q, np.zeros_like(kv), idx, sm_scale=0.2, d_v=Dv, k_scale=0.5,
                            attn_sink=sink, v8=kv[:, :Dv])
    b = A.sparse_attn_token(q, np.zeros_like(kv), idx, sm_scale=0.2, d_v=Dv, k_scale=7.0,
                            attn_sink=sink, v8=kv[:, :Dv])
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_q_k_sink_rescaling_invariance():
    q, kv, idx, sink, Dv = _tok_case(6)
    a = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, q_scale=0.75, k_scale=1.5, attn_sink=sink)
    b = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, q_scale=1.5, k_scale=0.75, attn_sink=sink / 2)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-12)


def test_v_scale_doubles_output_only():
    q, kv, idx, sink, Dv = _tok_case(7)
    a = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, v_scale=1.25, attn_sink=sink)
    b = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, v_scale=2.5, attn_sink=sink)
    assert np.array_equal(2 * a[0], b[0])
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_none_equals_unit_and_no_sink_equals_minus_inf():
    q, kv, idx, sink, Dv = _tok_case(8)
    a = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv)
    b = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, q_scale=1.0, k_scale=1.0, v_scale=1.0)
    c = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, attn_sink=np.full(q.shape[1], -np.inf))
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_permuting_index_list_is_invariant():
    q, kv, idx, sink, Dv = _tok_case(9)
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(r) for r in idx])
    a = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, attn_sink=sink)
    b = A.sparse_attn_token(q, kv, perm, sm_scale=0.2, d_v=Dv, attn_sink=sink)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-12)


def test_topk_length_truncates():
    q, kv, idx, sink, Dv = _tok_case(10)
    tl = np.array([40, 10, 1, 0, 25])
    a = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, d_v=Dv, topk_length=tl)
    cut = np.where(np.arange(idx.shape[1])[None] < tl[:, None], idx, -1)
    b = A.sparse_attn_token(q, kv, cut, sm_scale=0.2, d_v=Dv)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_token_mode_vs_library_masked_sdpa():
    q, kv, idx, sink, Dv = _tok_case(11)
    out, lse, _ = A.sparse_attn_token(q, kv, idx, sm_scale=0.2, q_scale=0.8, k_scale=1.3, v_scale=0.9, d_v=Dv)
    Q = torch.from_numpy(TAB[q]).transpose(0, 1)                # [H, T, D]
    K = torch.from_numpy(TAB[kv])[None]                         # [1, S, D]
    V = torch.from_numpy(TAB[kv[:, :Dv]])[None]
    mask = torch.zeros(q.shape[0], kv.shape[0], dtype=torch.bool)
    for t in range(q.shape[0]):
        mask[t, torch.from_numpy(idx[t])] = True
    scale = 0.2 * 0.8 * 1.3
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K.expand(Q.shape[0], -1, -1),
                                                           V.expand(Q.shape[0], -1, -1),
                                                           attn_mask=mask[None], scale=scale)
    assert np.allclose(out, 0.9 * ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    logits = scale * (Q @ K.transpose(1, 2))
    ref_lse = torch.logsumexp(logits.masked_fill(~mask[None], -math.inf), dim=-1).transpose(0, 1)
    assert np.allclose(lse, ref_lse.numpy(), atol=1e-10)


# ---------------------------------------------------------------- block mode

def _block_case(seq_len=700, Hq=8, Hkv=2, Hidx=4, D=16, Dv=16, seed=0, B=1, q_len=None):
    rng = np.random.default_rng(seed)
    q_len = seq_len if q_len is None else q_len
    nb = (seq_len + PAGE - 1) // PAGE
    P = B * nb + 2
    q = rand_codes(rng, (B * q_len, Hq, D))
    kc = rand_codes(rng, (P, Hkv, PAGE, D))
    vc = rand_codes(rng, (P, Hkv, PAGE, Dv))
    bt = rng.permutation(P)[: B * nb].reshape(B, nb).astype(np.int32)
    cu = (np.arange(B + 1) * q_len).astype(np.int32)
    sl = np.full(B, seq_len, np.int32)
    return q, kc, vc, bt, cu, sl


def test_block_mode_all_selected_equals_causal_sdpa():
    # every row has nb <= topk: the padding branch selects all causal blocks,
    # so block-sparse attention is ordinary causal attention (GQA)
    q, kc, vc, bt, cu, sl = _block_case(seq_len=600)
    T, Hq, D = q.shape
    Hkv = kc.shape[1]
    ids = np.stack([np.stack([IX.select_topk(np.zeros(t // PAGE + 1), 8) for t in range(T)])] * 4)
    toks = np.arange(0, T, 7)
    out, lse, mx = A.sparse_attn_block(q, kc, vc, ids, bt, cu, sl, sm_scale=0.25, q_scale=0.5,
                                       k_scale=1.5, v_scale=2.0, tokens=toks)
    # contiguous K/V in logical order for the library call
    K = TAB[kc[bt[0]]].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :T]
    V = TAB[vc[bt[0]]].transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :T]
    Q = TAB[q].transpose(1, 0, 2)                               # [Hq, T, D]
    Kx = torch.from_numpy(np.repeat(K, Hq // Hkv, axis=0))
    Vx = torch.from_numpy(np.repeat(V, Hq // Hkv, axis=0))
    scale = 0.25 * 0.5 * 1.5
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(Q), Kx, Vx, is_causal=True,
                                                           scale=scale)
    ref = 2.0 * ref.numpy().transpose(1, 0, 2)
    assert np.allclose(out, ref[toks], rtol=0, atol=1e-10)
    logits = scale * torch.from_numpy(Q) @ Kx.transpose(1, 2)
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(logits.masked_fill(~causal, -math.inf), dim=-1).numpy().T
    assert np.allclose(lse, ref_lse[toks], atol=1e-10)
    ref_mx = logits.masked_fill(~causal, -math.inf).amax(-1).numpy().T
    assert np.allclose(mx, ref_mx[toks], atol=1e-12)


def test_block_mode_selection_masks_unselected_blocks():
    # selecting blocks {0, 2} equals token mode over exactly those visible tokens
    q, kc, vc, bt, cu, sl = _block_case(seq_len=400, Hq=4, Hkv=1, Hidx=1, seed=3)
    T = q.shape[0]
    ids = np.full((1, T, 3), -1, np.int32)
    t = 390
    ids[0, t, :2] = [0, 2]
    out, lse, mx = A.sparse_attn_block(q, kc, vc, ids, bt, cu, sl, sm_scale=0.3, tokens=[t])
    keys = [j for j in range(t + 1) if j // PAGE in (0, 2)]
    kv_rows = np.stack([kc[bt[0, j // PAGE], 0, j % PAGE] for j in keys])
    v_rows = np.stack([vc[bt[0, j // PAGE], 0, j % PAGE] for j in keys])
    ref = A.sparse_attn_token(q[t:t + 1], kv_rows, np.arange(len(keys))[None], sm_scale=0.3,
                              d_v=v_rows.shape[1], v8=v_rows)
    assert np.allclose(out, ref[0], atol=1e-13) and np.allclose(lse, ref[1], atol=1e-13)


def test_block_mode_diagonal_block_is_causally_masked():
    q, kc, vc, bt, cu, sl = _block_case(seq_len=300, Hq=4, Hkv=1, Hidx=1, seed=4)
    T = q.shape[0]
    ids = np.full((1, T, 2), -1, np.int32)
    t = 200                    # block 1 holds tokens 128..255; only 128..200 visible
    ids[0, t, 0] = 1
    out, lse, mx = A.sparse_attn_block(q, kc, vc, ids, bt, cu, sl, sm_scale=0.3, tokens=[t])
    keys = list(range(128, 201))
    kv_rows = np.stack([kc[bt[0, 1], 0, j % PAGE] for j in keys])
    v_rows = np.stack([vc[bt[0, 1], 0, j % PAGE] for j in keys])
    ref = A.sparse_attn_token(q[t:t + 1], kv_rows, np.arange(len(keys))[None], sm_scale=0.3,
                              d_v=v_rows.shape[1], v8=v_rows)
    assert np.allclose(out, ref[0], atol=1e-13) and np.allclose(mx, ref[2], atol=1e-13)


def test_block_mode_head_mapping():
    # Hq=8, Hidx=4, Hkv=2: heads 0,1 -> idx 0, kv 0; heads 6,7 -> idx 3, kv 1
    q, kc, vc, bt, cu, sl = _block_case(seq_len=500, Hq=8, Hkv=2, Hidx=4, seed=5)
    T = q.shape[0]
    t = 450
    ids = np.full((4, T, 2), -1, np.int32)
    ids[0, t, 0] = 0
    ids[3, t, 0] = 2
    out, _, _ = A.sparse_attn_block(q, kc, vc, ids, bt, cu, sl, sm_scale=0.3, tokens=[t])
    for h, kvh, blk in ((0, 0, 0), (1, 0, 0), (6, 1, 2), (7, 1, 2)):
        keys = range(blk * PAGE, (blk + 1) * PAGE)
        kv_rows = np.stack([kc[bt[0, blk], kvh, j % PAGE] for j in keys])
        v_rows = np.stack([vc[bt[0, blk], kvh, j % PAGE] for j in keys])
        ref = A.sparse_attn_token(q[t:t + 1, h:h + 1], kv_rows, np.arange(PAGE)[None], sm_scale=0.3,
                                  d_v=v_rows.shape[1], v8=v_rows)
        assert np.allclose(out[0, h], ref[0][0, 0], atol=1e-13)
    for h in (2, 3, 4, 5):         # their index heads selected nothing
        assert np.all(out[0, h] == 0)


def test_block_mode_out_of_range_page_adds_no_keys():
    # ids {0, 1, 2} where block 1's table entry names no page (-1, then one past
    # the cache): the keys are those of blocks 0 and 2 only, as in token mode
    q, kc, vc, bt, cu, sl = _block_case(seq_len=400, Hq=4, Hkv=1, Hidx=1, seed=6)
    T = q.shape[0]
    t = 390
    ids = np.full((1, T, 3), -1, np.int32)
    ids[0, t] = [0, 1, 2]
    keys = [j for j in range(t + 1) if j // PAGE in (0, 2)]
    kv_rows = np.stack([kc[bt[0, j // PAGE], 0, j % PAGE] for j in keys])
    v_rows = np.stack([vc[bt[0, j // PAGE], 0, j % PAGE] for j in keys])
    ref = A.sparse_attn_token(q[t:t + 1], kv_rows, np.arange(len(keys))[None], sm_scale=0.3,
                              d_v=v_rows.shape[1], v8=v_rows)
    for bad in (-1, kc.shape[0]):
        bt2 = bt.copy()
        bt2[0, 1] = bad
        out, lse, mx = A.sparse_attn_block(q, kc, vc, ids, bt2, cu, sl, sm_scale=0.3, tokens=[t])
        assert np.allclose(out, ref[0], atol=1e-13) and np.allclose(lse, ref[1], atol=1e-13)
        assert np.allclose(mx, ref[2], atol=1e-13)
    # every selected block without a page: no keys at all
    bt3 = bt.copy()
    bt3[0, :3] = -1
    out, lse, mx = A.sparse_attn_block(q, kc, vc, ids, bt3, cu, sl, sm_scale=0.3, tokens=[t])
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(np.isneginf(mx))
