"""Sparse attention forward (test infrastructure only).

What the pages define
---------------------
* Only the selected KV tokens or blocks take part: QK dot, online softmax and
  PV product, with an optional per-head attention sink, a bf16 output and
  fp32 ``max_logits`` / ``lse`` of shape ``[s_q, h_q]`` (sglang PR 25751 digest,
  implementation step 1 and the ``sparse_mla_q8kv8_prefill_fwd`` code excerpt).
* Scale semantics: ``q_scale`` is folded into ``sm_scale`` so it multiplies both
  the QK dot and the sink logit, while ``k_scale`` never touches the sink term;
  ``v_scale`` applies to the output; ``None`` means unit scale (sglang PR 30971
  digest, summary and implementation step 3).
* MLA token mode: V is the first ``d_v = 512`` columns of the same KV row
  (sglang PR 25751 digest, code excerpt: the kernel hard-codes D_V = 512).
* Block mode: a query attends to the tokens of the blocks its index head
  selected; ascending ids with a ``-1`` tail (sglang PR 30971 digest,
  implementation step 2 and review thread 2).

Definition evaluated here (float64 on dequantized e4m3 inputs)::

    s       = sm_scale * q_scale
    z_j     = s * k_scale * <q, k_j>                 for j in the key set J
    z_sink  = s * sink[h]                             (if a sink is given)
    m       = max_j z_j            (-inf if J is empty)
    M       = max(m, z_sink)
    L       = sum_j exp(z_j - M) + [sink] exp(z_sink - M)
    out     = v_scale * sum_j exp(z_j - M) * v_j / L  (0 when L == 0)
    lse     = M + ln L             (-inf when L == 0)
    max_logits = m

Readings taken where the pages are silent: ``lse`` includes the sink and is a
natural log; ``max_logits`` is the maximum over key logits only.  Query head h
uses index head ``h // (Hq / Hidx)`` and KV head ``h // (Hq / Hkv)``.  In block
mode the key set is the union, over the row's ids ``0 <= b < max_blocks``, of
tokens ``128 b .. 128 b + 127`` that are ``<= p``; a block whose block-table
entry lies outside ``[0, num_pages)`` names no page and adds no key.  In token mode each valid
list entry (``0 <= idx < S``, within ``topk_length``) contributes one term.

Pins (tests/test_oracle_attention.py): closed forms (identical keys give
mean(V); one key gives V; one key plus a sink gives the logistic weight; the
sink-only limit gives 0), scale and sink invariants, permutation invariance,
and equality with torch's float64 causal scaled_dot_product_attention when a
block row selects every causal block.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import e4m3
from .indexer import positions


def _unit(s: Optional[float]) -> float:
    return 1.0 if s is None else float(s)


def softmax_rows(z: np.ndarray, vals: np.ndarray, z_sink: Optional[np.ndarray]):
    """Rows of logits z ``[R, n]`` against values ``[n, Dv]``.

    Returns (normalised output ``[R, Dv]``, lse ``[R]``, max_logits ``[R]``)
    with the definitions of the module docstring (v_scale not applied).
    """
    R = z.shape[0]
    if z.shape[1] == 0:
        m = np.full(R, -np.inf)
    else:
        m = z.max(axis=1)
    M = m.copy() if z_sink is None else np.maximum(m, z_sink)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.exp(z - Ms[:, None]) if z.shape[1] else np.zeros((R, 0))
    w = np.where(finite[:, None], w, 0.0)
    L = w.sum(axis=1)
    if z_sink is not None:
        L = L + np.where(finite, np.exp(z_sink - Ms), 0.0)
    num = w @ vals
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(L[:, None] > 0, num / np.where(L > 0, L, 1.0)[:, None], 0.0)
        lse = np.where(L > 0, M + np.log(np.where(L > 0, L, 1.0)), -np.inf)
    return out, lse, m


def sparse_attn_token(q8, kv8, indices, *, sm_scale: float, d_v: int,
                      q_scale: Optional[float] = None, k_scale: Optional[float] = None,
                      v_scale: Optional[float] = None, attn_sink=None, topk_length=None,
                      v8=None, tokens=None):
    """Token-index sparse attention (MLA style, one shared KV head).

    q8 ``[T, Hq, Dqk]`` codes, kv8 ``[S, Dqk]`` codes, indices ``[T, topk]``;
    V rows are ``kv8[:, :d_v]`` unless ``v8 [S, d_v]`` is given.
    Returns out ``[n, Hq, d_v]`` float64, lse ``[n, Hq]``, max_logits ``[n, Hq]``.
    """
    table = e4m3.decode_table()
    q8 = np.asarray(q8, dtype=np.uint8)
    kv8 = np.asarray(kv8, dtype=np.uint8)
    idx = np.asarray(indices, dtype=np.int64)
    T, Hq, _ = q8.shape
    S = kv8.shape[0]
    vsrc = kv8[:, :d_v] if v8 is None else np.asarray(v8, dtype=np.uint8)
    s = float(sm_scale) * _unit(q_scale)
    kscale = s * _unit(k_scale)
    vs = _unit(v_scale)
    sink = None if attn_sink is None else np.asarray(attn_sink, dtype=np.float64)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(toks), Hq, d_v))
    lse = np.zeros((len(toks), Hq))
    mx = np.zeros((len(toks), Hq))
    for r, t in enumerate(toks):
        row = idx[t]
        if topk_length is not None:
            row = row[: int(topk_length[t])]
        row = row[(row >= 0) & (row < S)]
        K = table[kv8[row]]                   # [n, Dqk]
        V = table[vsrc[row]]                  # [n, d_v]
        Q = table[q8[t]]                      # [Hq, Dqk]
        z = kscale * (Q @ K.T)                # [Hq, n]
        zs = None if sink is None else s * sink
        o, l, m = softmax_rows(z, V, zs)
        out[r] = vs * o
        lse[r] = l
        mx[r] = m
    return out, lse, mx


def sparse_attn_block(q8, k_cache8, v_cache8, ids, block_table, cu_seqlens_q, seq_lens, *,
                      sm_scale: float, q_scale: Optional[float] = None,
                      k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                      attn_sink=None, page_size: int = 128, tokens=None):
    """Block-sparse attention over paged K/V (GQA with nested index heads).

    q8 ``[T, Hq, D]``; k_cache8 ``[P, Hkv, page, D]``; v_cache8
    ``[P, Hkv, page, Dv]``; ids ``[Hidx, T, topk]``; block_table
    ``[B, max_blocks]``.  Returns out ``[n, Hq, Dv]``, lse ``[n, Hq]``,
    max_logits ``[n, Hq]`` (float64).
    """
    table = e4m3.decode_table()
    q8 = np.asarray(q8, dtype=np.uint8)
    kc = np.asarray(k_cache8, dtype=np.uint8)
    vc = np.asarray(v_cache8, dtype=np.uint8)
    ids = np.asarray(ids, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    T, Hq, D = q8.shape
    Hkv = kc.shape[1]
    Dv = vc.shape[3]
    Hidx = ids.shape[0]
    max_blocks = bt.shape[1]
    gq_idx = Hq // Hidx
    gq_kv = Hq // Hkv
    s = float(sm_scale) * _unit(q_scale)
    kscale = s * _unit(k_scale)
    vs = _unit(v_scale)
    sink = None if attn_sink is None else np.asarray(attn_sink, dtype=np.float64)
    seq, pos = positions(cu_seqlens_q, seq_lens)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(toks), Hq, Dv))
    lse = np.zeros((len(toks), Hq))
    mx = np.zeros((len(toks), Hq))
    for r, t in enumerate(toks):
        b, p = int(seq[t]), int(pos[t])
        Q = table[q8[t]]                      # [Hq, D]
        for g in range(Hidx):
            blocks = np.unique(ids[g, t])
            blocks = blocks[(blocks >= 0) & (blocks < max_blocks)]
            blocks = blocks[(bt[b, blocks] >= 0) & (bt[b, blocks] < kc.shape[0])]   # no page: no keys
            heads = np.arange(g * gq_idx, (g + 1) * gq_idx)
            for kvh in np.unique(heads // gq_kv):
                hs = heads[heads // gq_kv == kvh]
                if len(blocks):
                    kpos = (blocks[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)
                    keep = kpos <= p
                    pages = np.repeat(bt[b, blocks], page_size)[keep]
                    slots = (kpos % page_size)[keep]
                    K = table[kc[pages, kvh, slots]]           # [n, D]
                    V = table[vc[pages, kvh, slots]]           # [n, Dv]
                else:
                    K = np.zeros((0, D))
                    V = np.zeros((0, Dv))
                z = kscale * (Q[hs] @ K.T)
                zs = None if sink is None else s * sink[hs]
                o, l, m = softmax_rows(z, V, zs)
                out[r, hs] = vs * o
                lse[r, hs] = l
                mx[r, hs] = m
    return out, lse, mx
