"""Pins for the oracle's lightning indexer and ascending top-k (CPU only)."""

import numpy as np
import pytest

from oracle import e4m3
from oracle import indexer as IX
from workloads import E4M3_EXACT_INTS, e4m3_codes

PAGE = 128


def tiny_case(seq_len=1000, q_len=None, H=2, D=16, seed=0, B=1, exact=True):
    rng = np.random.default_rng(seed)
    q_len = seq_len if q_len is None else q_len
    nb = (seq_len + PAGE - 1) // PAGE
    P = B * nb + 3
    T = B * q_len
    if exact:
        qv = rng.choice(E4M3_EXACT_INTS, (T, H, D)) * rng.choice([-1.0, 1.0], (T, H, D))
        kv = rng.choice(E4M3_EXACT_INTS[E4M3_EXACT_INTS <= 16], (P, PAGE, D)) * rng.choice([-1.0, 1.0], (P, PAGE, D))
    else:
        qv = rng.standard_normal((T, H, D))
        kv = rng.standard_normal((P, PAGE, D))
    q8 = e4m3_codes(qv.astype(np.float32))
    k8 = e4m3_codes(kv.astype(np.float32))
    bt = rng.permutation(P)[: B * nb].reshape(B, nb).astype(np.int32)
    cu = (np.arange(B + 1) * q_len).astype(np.int32)
    sl = np.full(B, seq_len, np.int32)
    return q8, k8, bt, cu, sl


def brute_row(q8, k8, bt, cu, sl, t, h, sigma, topk):
    """Independent per-token loop: scores every visible token one at a time."""
    tab = e4m3.decode_table()
    b = int(np.searchsorted(cu, t, side="right") - 1)
    q_len = int(cu[b + 1] - cu[b])
    p = int(sl[b]) - q_len + (t - int(cu[b]))
    nb = p // PAGE + 1
    best = {blk: -np.inf for blk in range(nb)}    # a block whose page is missing keeps -inf
    for j in range(p + 1):
        page = int(bt[b, j // PAGE])
        if page < 0 or page >= k8.shape[0]:
            continue                                # no page: the block holds no key
        dot = 0.0
        for d in range(q8.shape[2]):
            dot += tab[q8[t, h, d]] * tab[k8[page, j % PAGE, d]]
        s = sigma * dot
        blk = j // PAGE
        best[blk] = max(best[blk], s)
    if nb <= topk:
        return list(range(nb)) + [-1] * (topk - nb)
    items = sorted(best.items(), key=lambda kv: (-kv[1], kv[0]))[:topk]
    return sorted(k for k, _ in items)


def check_contract(ids, nbs, topk):
    for row, nb in zip(ids, nbs):
        if nb <= topk:
            assert list(row) == list(range(nb)) + [-1] * (topk - nb)
        else:
            assert np.all(row >= 0) and np.all(np.diff(row) > 0) and row[-1] < nb


def test_padding_branch_closed_form():
    q8, k8, bt, cu, sl = tiny_case(seq_len=700)
    ids = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.1, topk=8)
    _, pos = IX.positions(cu, sl)
    for t in range(0, 700, 37):
        nb = pos[t] // PAGE + 1
        assert list(ids[0, t]) == list(range(nb)) + [-1] * (8 - nb)


@pytest.mark.parametrize("topk", [1, 2, 3, 5])
def test_brute_force_rows(topk):
    q8, k8, bt, cu, sl = tiny_case(seq_len=900, D=8, seed=topk)
    sigma = 0.3 * 1.7 * 0.6
    ids = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.3, idx_q_scale=1.7, idx_k_scale=0.6, topk=topk)
    for t in (0, 127, 128, 300, 511, 777, 899):
        for h in range(2):
            assert list(ids[h, t]) == brute_row(q8, k8, bt, cu, sl, t, h, sigma, topk), (t, h)


def test_planted_permutation():
    # one-hot index query on dim 0; key dim 0 encodes a per-block value, so the
    # block maxima are a known permutation and the answer is known in advance
    rng = np.random.default_rng(3)
    nb, D, T = 10, 8, 10 * PAGE
    q = np.zeros((T, 1, D), np.float32)
    q[:, 0, 0] = 1.0
    vals = rng.permutation(np.arange(1, nb + 1)).astype(np.float32)   # distinct, exact
    k = np.zeros((nb, PAGE, D), np.float32)
    k[:, :, 0] = -1.0
    k[:, 0, 0] = vals          # first token of each block carries the block max
    bt = np.arange(nb, dtype=np.int32)[None]
    cu = np.array([0, T], np.int32)
    sl = np.array([T], np.int32)
    ids = IX.indexer_topk(e4m3_codes(q), e4m3_codes(k), bt, cu, sl, sm_scale=1.0, topk=4)
    expect = np.sort(np.argsort(-vals, kind="stable")[:4])
    assert list(ids[0, T - 1]) == list(expect)
    # a token that sees 6 blocks only chooses among those
    t = 5 * PAGE
    expect6 = np.sort(np.argsort(-vals[:6], kind="stable")[:4])
    assert list(ids[0, t]) == list(expect6)


def test_ties_break_to_lower_id():
    nb, D, T = 6, 4, 6 * PAGE
    q = np.zeros((T, 1, D), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((nb, PAGE, D), np.float32)
    k[:, :, 0] = 2.0           # every block ties
    bt = np.arange(nb, dtype=np.int32)[None]
    ids = IX.indexer_topk(e4m3_codes(q), e4m3_codes(k), bt, np.array([0, T], np.int32),
                          np.array([T], np.int32), sm_scale=1.0, topk=3)
    assert list(ids[0, T - 1]) == [0, 1, 2]


def test_scale_invariance_of_ids():
    q8, k8, bt, cu, sl = tiny_case(seq_len=1500, D=16, seed=11)
    a = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=1.0, topk=4)
    b = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.088, idx_q_scale=3.1, idx_k_scale=0.17, topk=4)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("topk", [16, 32, 33, 48, 64])
def test_k_sweep_contract_and_brute_force(topk):
    # long enough that rows near the end have more than topk blocks
    L = (topk + 6) * PAGE
    q8, k8, bt, cu, sl = tiny_case(seq_len=L, q_len=3, H=1, D=4, seed=topk)
    ids = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.5, topk=topk)
    _, pos = IX.positions(cu, sl)
    check_contract(ids[0], pos // PAGE + 1, topk)
    for t in range(3):
        assert list(ids[0, t]) == brute_row(q8, k8, bt, cu, sl, t, 0, 0.5, topk)


def test_varlen_positions_and_decode():
    # two sequences with prefixes: positions follow seq_len - q_len + i
    cu = np.array([0, 3, 4], np.int32)
    sl = np.array([10, 300], np.int32)
    seq, pos = IX.positions(cu, sl)
    assert list(seq) == [0, 0, 0, 1]
    assert list(pos) == [7, 8, 9, 299]


def test_out_of_range_pages_hold_no_keys():
    """A block-table entry outside [0, num_pages) names no page: its block has
    no key and scores -inf, below every block with a key, but stays a
    candidate (lowest ids first among such blocks)."""
    q8, k8, bt, cu, sl = tiny_case(seq_len=1280, D=8, seed=5)
    P = k8.shape[0]
    bt = bt.copy()
    bt[0, [2, 5, 7]] = [-1, P, P + 40]              # three blocks without a page
    sc = IX.block_scores(q8, k8, bt, cu, sl, sm_scale=0.25, tokens=[1279])[0]
    assert np.all(np.isneginf(sc[:, [2, 5, 7]])) and np.all(np.isfinite(np.delete(sc, [2, 5, 7], axis=1)))
    # 10 visible blocks, 7 with keys: top-4 picks among the 7 only
    ids = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.25, topk=4)
    for t in (700, 1000, 1279):
        for h in range(2):
            row = list(ids[h, t])
            assert not set(row) & {2, 5, 7}
            assert row == brute_row(q8, k8, bt, cu, sl, t, h, 0.25, 4), (t, h)
    # top-8 of the 10: all 7 blocks with keys, then the lowest id without one
    ids8 = IX.indexer_topk(q8, k8, bt, cu, sl, sm_scale=0.25, topk=8)
    assert list(ids8[0, 1279]) == [0, 1, 2, 3, 4, 6, 8, 9]
    assert list(ids8[1, 1279]) == brute_row(q8, k8, bt, cu, sl, 1279, 1, 0.25, 8)
