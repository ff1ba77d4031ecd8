"""Lightning-indexer block scoring and ascending top-k (test infrastructure only).

What the pages define
---------------------
* Each 128-token KV block is scored against the index query; the prefill
  scorer returns one maximum score per 128-wide tile and the tile id is the
  block id (vLLM PR 45892 digest, implementation step 1 and the code excerpt's
  ``PAGE_SIZE`` comment).
* The index query is ``[total_q, H, 128]``, the index-key cache is
  ``[num_pages, 128, 128]`` (one head) and a block table maps logical blocks
  to physical pages (same digest, code excerpt of ``_fmha_indexer_topk``).
* The selected ids are written strictly ascending; when a row has no more
  blocks than k, ids ``0..nb-1`` are written followed by ``-1`` padding, and
  that branch never overlaps the selecting branch (sglang PR 30971 digest,
  implementation step 2 and review thread 2).
* One selection per index head per token: the shared buffer is
  ``[num_index_heads, max_num_batched_tokens, topk_blocks]`` (vLLM PR 45892
  digest, implementation step 4).

Readings taken where the pages are silent
-----------------------------------------
* Query position: ``p = seq_lens[b] - q_len_b + i`` for the i-th query of
  sequence b (seq_lens include the current step: keys are stored before the
  indexer runs).  Key j is visible iff ``j <= p``.
* Block score: ``S[h, t, b] = max_{j in block b, j <= p} sigma * <iq[t,h], ik[j]>``
  with ``sigma = sm_scale * idx_q_scale * idx_k_scale`` (each scale ``None``
  means 1).  Plain maximum: no ReLU, no sum, no cross-head weighting.
* Ties: larger score first, then the lower block id.  No forced blocks.
* A block-table entry outside ``[0, num_pages)`` names no page: that block
  holds no key, so its score is the maximum over an empty set, ``-inf``.  It
  still counts among the ``nb`` visible blocks and stays a candidate, ranked
  below every block that has a key (ties among such blocks go to the lower
  id, as any tie does).

Everything is float64 on dequantized e4m3 inputs; selection is a brute-force
sort.

Pins (tests/test_oracle_indexer.py): the padding branch's closed form, a
planted permutation of block maxima, invariance of ids to positive scales, a
brute-force recomputation of one row through an independent per-token loop,
and the structural contract (ascending, distinct, -1 only at the tail).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import e4m3


def _unit(s: Optional[float]) -> float:
    return 1.0 if s is None else float(s)


def positions(cu_seqlens_q, seq_lens) -> tuple[np.ndarray, np.ndarray]:
    """(sequence id, absolute position p) of every flattened query token."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    T = int(cu[-1])
    seq = np.zeros(T, dtype=np.int64)
    pos = np.zeros(T, dtype=np.int64)
    for b in range(len(sl)):
        q_len = int(cu[b + 1] - cu[b])
        seq[cu[b]:cu[b + 1]] = b
        pos[cu[b]:cu[b + 1]] = sl[b] - q_len + np.arange(q_len)
    return seq, pos


def block_scores(idx_q8, idx_k8, block_table, cu_seqlens_q, seq_lens, *, sm_scale: float,
                 idx_q_scale: Optional[float] = None, idx_k_scale: Optional[float] = None,
                 page_size: int = 128, tokens=None, chunk: int = 64) -> list[np.ndarray]:
    """Float64 block scores.  Returns one ``[H, nb_t]`` array per requested token."""
    q = np.asarray(idx_q8, dtype=np.uint8)
    T, H, D = q.shape
    kc = np.asarray(idx_k8, dtype=np.uint8)
    bt = np.asarray(block_table, dtype=np.int64)
    sigma = float(sm_scale) * _unit(idx_q_scale) * _unit(idx_k_scale)
    seq, pos = positions(cu_seqlens_q, seq_lens)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    table = e4m3.decode_table()
    result: list[np.ndarray] = [None] * len(toks)  # type: ignore[list-item]

    # group requested tokens by sequence so that each sequence's keys are decoded once
    for b in np.unique(seq[toks]):
        sel = np.nonzero(seq[toks] == b)[0]
        pmax = int(pos[toks[sel]].max())
        nb_max = pmax // page_size + 1
        pages = bt[b, :nb_max]
        has_page = (pages >= 0) & (pages < kc.shape[0])
        keys = table[kc[np.where(has_page, pages, 0)]]   # [nb_max, page, D]; rows of absent pages are masked
        key_pos = np.arange(nb_max * page_size).reshape(nb_max, page_size)
        for c0 in range(0, len(sel), chunk):
            ids = sel[c0:c0 + chunk]
            tt = toks[ids]
            qv = table[q[tt]]                        # [n, H, D]
            dots = np.einsum("nhd,bpd->nhbp", qv, keys, optimize=True) * sigma
            vis = key_pos[None, :, :] <= pos[tt][:, None, None]     # [n, nb_max, page]
            vis = vis & has_page[None, :, None]                     # a block without a page has no key
            dots = np.where(vis[:, None, :, :], dots, -np.inf)
            s = dots.max(axis=3)                     # [n, H, nb_max]
            for r, i in enumerate(ids):
                nb = int(pos[toks[i]]) // page_size + 1
                result[i] = s[r, :, :nb].copy()
    return result


def select_topk(scores: np.ndarray, topk: int) -> np.ndarray:
    """Ascending top-k ids of one row of block scores (``nb`` entries)."""
    nb = scores.shape[0]
    if nb <= topk:
        return np.concatenate([np.arange(nb), -np.ones(topk - nb, dtype=np.int64)]).astype(np.int32)
    ids = np.arange(nb)
    order = np.lexsort((ids, -scores))             # by score descending, then id ascending
    return np.sort(order[:topk]).astype(np.int32)


def indexer_topk(idx_q8, idx_k8, block_table, cu_seqlens_q, seq_lens, *, sm_scale: float,
                 topk: int, idx_q_scale: Optional[float] = None,
                 idx_k_scale: Optional[float] = None, page_size: int = 128,
                 tokens=None) -> np.ndarray:
    """Top-k block ids, ``[H, n_tokens, topk]`` int32, ascending with -1 tail.

    Rows whose block count does not exceed ``topk`` take the closed-form
    padding branch without scoring.
    """
    q = np.asarray(idx_q8, dtype=np.uint8)
    T, H, _ = q.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    _, pos = positions(cu_seqlens_q, seq_lens)
    out = np.empty((H, len(toks), topk), dtype=np.int32)
    need = [i for i, t in enumerate(toks) if int(pos[t]) // page_size + 1 > topk]
    for i, t in enumerate(toks):
        nb = int(pos[t]) // page_size + 1
        if nb <= topk:
            out[:, i, :] = select_topk(np.zeros(nb), topk)
    if need:
        sc = block_scores(q, idx_k8, block_table, cu_seqlens_q, seq_lens, sm_scale=sm_scale,
                          idx_q_scale=idx_q_scale, idx_k_scale=idx_k_scale,
                          page_size=page_size, tokens=toks[need])
        for j, i in enumerate(need):
            for h in range(H):
                out[h, i, :] = select_topk(sc[j][h], topk)
    return out
