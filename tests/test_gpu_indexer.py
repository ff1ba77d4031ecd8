"""indexer_topk on the GPU vs the oracle: bit-exact ids.

Exact-mode inputs (index codes that are e4m3-exact integers, |q| <= 64,
|k| <= 16) make every index dot product an integer below 2^17, exact in fp32
under any summation order, so the GPU must reproduce the oracle's ids bit for
bit, ties included.  N(0,1) inputs are checked for set validity within the
fp32 rounding bound instead.
"""

import numpy as np
import pytest
import torch

from oracle import indexer as OI
from oracle import quantize as OQ
import workloads as W
from helpers import bf16_dev, dev, exact_workload_ids, host, scores_margin_ok, workload

pytestmark = pytest.mark.gpu
PAGE = 128


def exact_codes(rng, shape, kmax):
    vals = W.E4M3_EXACT_INTS[W.E4M3_EXACT_INTS <= kmax]
    v = rng.choice(vals, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    return W.e4m3_codes(v.astype(np.float32))


def make_case(seq_lens, q_lens, seed, H=4, extra_pages=3):
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    nbs = [(s + PAGE - 1) // PAGE for s in seq_lens]
    max_blocks = max(nbs)
    P = sum(nbs) + extra_pages
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((B, max_blocks), -1, np.int32)
    o = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[o:o + nb]
        o += nb
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    iq = exact_codes(rng, (T, H, 128), 64)
    ik = exact_codes(rng, (P, PAGE, 128), 16)
    return iq, ik, bt, cu, np.asarray(seq_lens, np.int32), max(q_lens)


def run(gpu, iq, ik, bt, cu, sl, mq, topk, sm=0.088, qs=None, ks=None):
    return host(gpu.indexer_topk(dev(iq), dev(ik), dev(bt), dev(cu), dev(sl), max_q_len=mq, sm_scale=sm,
                                 topk=topk, idx_q_scale=qs, idx_k_scale=ks))


def assert_ids_equal(got, ref, what):
    bad = np.argwhere(np.any(got != ref, axis=2))
    assert bad.size == 0, f"{what}: {len(bad)} rows differ, first (h, t) {bad[:4].tolist()}"


@pytest.mark.parametrize("topk", [4, 8])
def test_prefill_exact(gpu, topk):
    iq, ik, bt, cu, sl, mq = make_case([3000], [3000], seed=topk)
    got = run(gpu, iq, ik, bt, cu, sl, mq, topk, qs=2.5, ks=0.3)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, idx_q_scale=2.5, idx_k_scale=0.3, topk=topk)
    assert_ids_equal(got, ref, "prefill")


@pytest.mark.parametrize("topk", [16, 32, 33, 48, 64])
def test_k_sweep(gpu, topk):
    L = (topk + 9) * PAGE + 17
    iq, ik, bt, cu, sl, mq = make_case([L], [L], seed=100 + topk, H=4)
    got = run(gpu, iq, ik, bt, cu, sl, mq, topk)
    toks = np.arange(L - 200, L)              # rows with more blocks than k
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=topk, tokens=toks)
    assert_ids_equal(got[:, toks], ref, f"k={topk}")
    # the padding branch for every earlier row
    _, pos = OI.positions(cu, sl)
    for t in range(0, L - 200, 97):
        nb = pos[t] // PAGE + 1
        if nb <= topk:
            assert list(got[0, t]) == list(range(nb)) + [-1] * (topk - nb)


def test_varlen_prefix_and_decode_mix(gpu):
    # sequence 0: prefill with a 1100-token prefix; 1: plain prefill; 2, 3: decode
    iq, ik, bt, cu, sl, mq = make_case([1700, 900, 5000, 129], [600, 900, 1, 1], seed=3, H=4)
    got = run(gpu, iq, ik, bt, cu, sl, mq, 5)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=5)
    assert_ids_equal(got, ref, "varlen")


@pytest.mark.parametrize("topk", [40, 41])
def test_varlen_closed_form_when_no_row_exceeds_k(gpu, topk):
    """max_blocks <= k: every row is the closed form 0 .. nb-1, -1 ... (varlen
    with a prefix, plain prefill and decode rows)."""
    iq, ik, bt, cu, sl, mq = make_case([5000, 1300, 128, 4097], [700, 1300, 1, 1], seed=40, H=4)
    assert bt.shape[1] <= topk
    got = run(gpu, iq, ik, bt, cu, sl, mq, topk)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=topk)
    assert_ids_equal(got, ref, f"closed form k={topk}")


@pytest.mark.parametrize("H", [1, 2, 8, 16])
def test_head_counts(gpu, H):
    iq, ik, bt, cu, sl, mq = make_case([1500, 700], [300, 700], seed=H, H=H)
    got = run(gpu, iq, ik, bt, cu, sl, mq, 3)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=3)
    assert_ids_equal(got, ref, f"H={H}")


def test_decode_batch_exact(gpu):
    rng = np.random.default_rng(9)
    seq = [int(x) for x in rng.integers(1, 20000, 24)] + [1, 128, 129, 64 * 128, 64 * 128 + 1]
    iq, ik, bt, cu, sl, mq = make_case(seq, [1] * len(seq), seed=10, H=4)
    got = run(gpu, iq, ik, bt, cu, sl, mq, 64)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=64)
    assert_ids_equal(got, ref, "decode")


@pytest.mark.parametrize("q_lens", [[2000], [1]])
def test_pages_outside_the_cache_hold_no_keys(gpu, q_lens):
    """Block-table entries outside [0, num_pages) (-1, one past the cache, far
    past it) name no page: those blocks score -inf against the oracle's rule,
    in the prefill (2000 queries) and decode (1 query) score kernels."""
    iq, ik, bt, cu, sl, mq = make_case([2000], q_lens, seed=4 + len(q_lens) + q_lens[0])
    P = ik.shape[0]
    bt = bt.copy()
    bt[0, [3, 7, 11]] = [-1, P, 10_000_000]
    for topk in (4, 13):       # 16 blocks, 13 with keys: k = 13 leaves no room for the three
        got = run(gpu, iq, ik, bt, cu, sl, mq, topk)
        ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=topk)
        assert_ids_equal(got, ref, f"absent pages k={topk}")
        assert not np.isin(got[:, -1], [3, 7, 11]).any()
    # k = 15 of 16: all 13 blocks with keys, then the two lowest ids without one
    got = run(gpu, iq, ik, bt, cu, sl, mq, 15)
    ref = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.088, topk=15)
    assert_ids_equal(got, ref, "absent pages k=15")
    assert list(got[0, -1]) == [b for b in range(16) if b != 11]


def test_prefill_32k_exact_full(gpu):
    """Full-size 32k prefill indexer (exact-mode codes, U(0.1,4) scales): every
    one of the 4 x 32768 id rows bit-exact against the oracle."""
    wl = workload(3)
    iq, ik, ref = exact_workload_ids(3)
    got = run(gpu, iq, ik, wl.block_table, wl.cu_seqlens_q, wl.seq_lens, wl.max_q_len, wl.topk,
              sm=wl.idx_sm_scale, qs=wl.idx_q_scale, ks=wl.idx_k_scale)
    assert_ids_equal(got, ref, "32k full")


def test_decode_64x32k_exact_full(gpu):
    """Full-size decode indexer: 64 sequences x 32768 tokens, exact-mode codes,
    all 4 x 64 id rows bit-exact against the oracle."""
    wl = workload(5)
    iq, ik, ref = exact_workload_ids(5)
    got = run(gpu, iq, ik, wl.block_table, wl.cu_seqlens_q, wl.seq_lens, wl.max_q_len, wl.topk,
              sm=wl.idx_sm_scale, qs=wl.idx_q_scale, ks=wl.idx_k_scale)
    assert_ids_equal(got, ref, "decode full")
    assert np.all(np.diff(got, axis=2) > 0)


def test_prefill_8k_padding_branch_full(gpu):
    """8k prefill: every row has <= 64 blocks, so the ids are the closed form."""
    wl = workload(2)
    q8 = OQ.quantize(wl.idx_q_bf16, OQ.BF16, wl.idx_q_scale)
    got = run(gpu, q8, wl.idx_k8, wl.block_table, wl.cu_seqlens_q, wl.seq_lens, wl.max_q_len, wl.topk,
              sm=wl.idx_sm_scale)
    T = wl.q_bf16.shape[0]
    nb = np.arange(T) // PAGE + 1
    ref = np.where(np.arange(64)[None, :] < nb[:, None], np.arange(64)[None, :], -1)
    for h in range(4):
        assert np.array_equal(got[h], ref)


@pytest.mark.parametrize("n", [3, 5])
def test_normal_inputs_set_validity(gpu, n):
    """N(0,1) codes: selection valid within the fp32 accumulation bound."""
    wl = workload(n)
    q8 = OQ.quantize(wl.idx_q_bf16, OQ.BF16, wl.idx_q_scale)
    got = run(gpu, q8, wl.idx_k8, wl.block_table, wl.cu_seqlens_q, wl.seq_lens, wl.max_q_len, wl.topk,
              sm=wl.idx_sm_scale, qs=wl.idx_q_scale, ks=wl.idx_k_scale)
    T = q8.shape[0]
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(T, min(T, 24), replace=False))
    sc = OI.block_scores(q8, wl.idx_k8, wl.block_table, wl.cu_seqlens_q, wl.seq_lens,
                         sm_scale=wl.idx_sm_scale, idx_q_scale=wl.idx_q_scale,
                         idx_k_scale=wl.idx_k_scale, tokens=toks)
    from oracle import e4m3
    tab = e4m3.decode_table()
    sigma = wl.idx_sm_scale * (wl.idx_q_scale or 1.0) * (wl.idx_k_scale or 1.0)
    present = np.nonzero(np.bincount(wl.idx_k8.reshape(-1), minlength=256))[0]
    kmax = np.nanmax(np.abs(tab[present]))
    for j, t in enumerate(toks):
        for h in range(4):
            qa = np.abs(tab[q8[t, h]]).sum()
            eps = 2 * 128 * 2.0 ** -24 * qa * kmax * sigma * 4
            assert scores_margin_ok(got[h, t], sc[j][h], wl.topk, eps), (t, h)
