"""Shared helpers for the GPU parity tests (inputs to device, comparisons)."""

from __future__ import annotations

import math

import numpy as np
import torch

# acceptance tolerances for floating-point outputs
OUT_RTOL = 2e-2     # max|out - ref| <= OUT_RTOL * max|ref|
LSE_ATOL = 1e-3     # |lse - ref| <= LSE_ATOL
ML_TOL = 1e-3       # |max_logits - ref| <= ML_TOL * max(1, |ref|)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def assert_attention_close(gpu, ref, what=""):
    out, ml, lse = (host(x) for x in gpu)
    r_out, r_lse, r_ml = ref
    scale = max(np.abs(r_out).max(), 1e-30)
    err = np.abs(out - r_out).max()
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    assert err <= OUT_RTOL * scale, f"{what}: max|err| {err:.3e} > {OUT_RTOL} * {scale:.3e}"
    # lse: -inf must match -inf exactly, finite values within LSE_ATOL
    assert np.array_equal(np.isneginf(lse), np.isneginf(r_lse)), f"{what}: lse -inf pattern differs"
    fin = np.isfinite(r_lse)
    if fin.any():
        e = np.abs(lse[fin] - r_lse[fin]).max()
        assert e <= LSE_ATOL, f"{what}: lse err {e:.3e}"
    assert np.array_equal(np.isneginf(ml), np.isneginf(r_ml)), f"{what}: max_logits -inf pattern differs"
    fin = np.isfinite(r_ml)
    if fin.any():
        e = (np.abs(ml[fin] - r_ml[fin]) / np.maximum(1.0, np.abs(r_ml[fin]))).max()
        assert e <= ML_TOL, f"{what}: max_logits rel err {e:.3e}"
    return err / scale


def scores_margin_ok(ids_row, scores_row, topk, eps):
    """Set validity for non-exact inputs: every selected block's score is at
    least every unselected block's score minus eps."""
    nb = len(scores_row)
    if nb <= topk:
        return list(ids_row) == list(range(nb)) + [-1] * (topk - nb)
    sel = np.asarray(ids_row)
    if np.any(sel < 0) or np.any(np.diff(sel) <= 0) or sel[-1] >= nb:
        return False
    mask = np.zeros(nb, bool)
    mask[sel] = True
    return scores_row[mask].min() >= scores_row[~mask].max() - eps


def causal_index_flops(ids: np.ndarray, seq_lens, cu, Hq: int, Hidx: int, d_qk: int, d_v: int, page=128):
    """Exact algorithmic flops of block-sparse attention (2 (d_qk + d_v) per visible key)."""
    H, T, k = ids.shape
    cu = np.asarray(cu)
    sl = np.asarray(seq_lens)
    total = 0
    for b in range(len(sl)):
        for t in range(cu[b], cu[b + 1]):
            p = sl[b] - (cu[b + 1] - cu[b]) + (t - cu[b])
            for g in range(H):
                blks = np.unique(ids[g, t])
                blks = blks[blks >= 0]
                n = np.minimum(p + 1 - blks * page, page).clip(min=0).sum()
                total += int(n) * (Hq // Hidx)
    return total * 2 * (d_qk + d_v)


def nan_safe_max(a):
    a = np.asarray(a)
    return -math.inf if a.size == 0 else float(np.nanmax(a))


_WL_CACHE = {}


def workload(n: int):
    """Cached full-size workload ``n`` (generation of the large ones takes seconds)."""
    import workloads as W
    if n not in _WL_CACHE:
        _WL_CACHE[n] = W.workload(n)
    return _WL_CACHE[n]


_IDS_CACHE = {}


def exact_workload_ids(n: int):
    """(exact-mode index query codes, index-key codes, oracle ids [Hidx, T, k])
    of full-size block workload ``n`` (3: 32k prefill, 5: 64 x 32k decode),
    every row computed by the oracle and cached for the session (about 20 s
    of float64 scoring for the 32k prompt)."""
    import workloads as W
    from oracle import indexer as OI
    if n not in _IDS_CACHE:
        wl = workload(n)
        if "idx_q8_exact" in wl.extra:
            iq, ik = wl.extra["idx_q8_exact"], wl.extra["idx_k8_exact"]
        else:
            iq, ik = W.exact_index_codes(1000 + n, wl.idx_q_bf16.shape[0], wl.idx_q_bf16.shape[1],
                                         wl.idx_q_bf16.shape[2], wl.idx_k8.shape[0])
        ids = OI.indexer_topk(iq, ik, wl.block_table, wl.cu_seqlens_q, wl.seq_lens, sm_scale=wl.idx_sm_scale,
                              idx_q_scale=wl.idx_q_scale, idx_k_scale=wl.idx_k_scale, topk=wl.topk)
        _IDS_CACHE[n] = (iq, ik, ids)
    return _IDS_CACHE[n]
