"""Seeded synthetic inputs for the five FP8 top-k sparse attention workloads.

This module only draws random numbers and stores them in the input formats
(bf16 bit patterns for activations, e4m3fn byte codes for caches, int32 index
lists and block tables).  It holds none of the method's arithmetic: no
quantization scale is applied, nothing is scored, selected or attended.  The
format casts use torch's CPU casts (float32 -> bfloat16 and
float32 -> float8_e4m3fn, both round-to-nearest-even), i.e. library
conversions, not this project's code.  Both the HIP path's tests and the CPU
oracle read the very same arrays.

Recipe (numpy PCG64, ``seed = 1000 + workload number``), draws in this order:
Q, idx_q, K/V (or KV), idx_k, scales, sink, token index lists, block-table
permutation.  Activations are N(0,1) in fp32 rounded to bf16; a cache with
per-tensor scale s stores codes of N(0, 1/s^2) draws, so that
``s * dequant(code)`` is N(0,1) like the activations it came from (the
"stored value = x / scale" convention).

Workloads (sizes are those of the method's long-context serving setting, one
GPU's head share):

1. tiny MLA token-sparse prefill: 64 queries x 16 heads, d_qk 576 / d_v 512,
   4096 KV rows, 256 distinct indices per query, scales q 0.5 k 0.25 v 2.0,
   per-head sink.
2. GQA block-sparse causal prefill, 8192 tokens, 16 q / 2 kv heads, d 128,
   page 128, indexer 4 heads x 128, top-64 blocks, unit scales.
3. as 2 at 32768 tokens with q/k/v/idx_q/idx_k scales drawn U(0.1, 4).
4. long MLA token-sparse prefill: 4096 queries x 128 heads over 65536 KV rows,
   top-2048 indices per query, sink, unit scales.
5. block-sparse decode: 64 sequences x 32768 tokens, q_len 1, paged caches,
   16 q / 2 kv heads, indexer 4 heads, top-64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAGE = 128

# Integers exactly representable in e4m3 (the index-test construction that makes
# fp8 and wide scores choose the same blocks): 1..16, then step 2 to 32, step 4 to 64.
E4M3_EXACT_INTS = np.array(list(range(0, 17)) + list(range(18, 33, 2)) + list(range(36, 65, 4)),
                           dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) by torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 array -> e4m3fn byte codes by torch's RNE cast (|x| must stay < 448)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _normal_codes(rng: np.random.Generator, shape, std: float = 1.0, chunk: int = 1 << 26) -> np.ndarray:
    """e4m3 codes of N(0, std^2) draws, generated in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = e4m3_codes(rng.normal(0.0, std, size=m).astype(np.float32))
    return out.reshape(shape)


def _distinct_sorted(rng: np.random.Generator, rows: int, k: int, n: int) -> np.ndarray:
    out = np.empty((rows, k), dtype=np.int32)
    for r in range(rows):
        out[r] = np.sort(rng.choice(n, size=k, replace=False))
    return out


@dataclass
class TokenWorkload:
    """MLA-style token-sparse prefill inputs (one shared KV head)."""
    name: str
    q_bf16: np.ndarray          # uint16 [T, Hq, Dqk]
    kv8: np.ndarray             # uint8  [S, Dqk]
    indices: np.ndarray         # int32  [T, topk]
    sink: Optional[np.ndarray]  # float32 [Hq]
    sm_scale: float
    d_v: int
    q_scale: Optional[float]
    k_scale: Optional[float]
    v_scale: Optional[float]
    topk_length: Optional[np.ndarray] = None


@dataclass
class BlockWorkload:
    """MiniMax-style GQA block-sparse inputs (prefill or decode)."""
    name: str
    q_bf16: np.ndarray          # uint16 [T, Hq, D]
    idx_q_bf16: np.ndarray      # uint16 [T, Hidx, Didx]
    k_cache8: np.ndarray        # uint8 [P, Hkv, PAGE, D]
    v_cache8: np.ndarray        # uint8 [P, Hkv, PAGE, D]
    idx_k8: np.ndarray          # uint8 [P, PAGE, Didx]
    block_table: np.ndarray     # int32 [B, max_blocks]
    cu_seqlens_q: np.ndarray    # int32 [B+1]
    seq_lens: np.ndarray        # int32 [B]
    max_q_len: int
    topk: int
    sm_scale: float
    idx_sm_scale: float
    q_scale: Optional[float]
    k_scale: Optional[float]
    v_scale: Optional[float]
    idx_q_scale: Optional[float]
    idx_k_scale: Optional[float]
    sink: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def _sink_for(rng: np.random.Generator, heads: int, n_keys: int, sm: float, q_scale: float) -> np.ndarray:
    # effective sink logit ln(n_keys) + N(0,1), passed in pre-scale units
    z = math.log(n_keys) + rng.standard_normal(heads)
    return (z / (sm * q_scale)).astype(np.float32)


def token_workload(T: int, Hq: int, S: int, topk: int, *, seed: int, name: str,
                   q_scale=None, k_scale=None, v_scale=None, with_sink=True,
                   d_qk: int = 576, d_v: int = 512) -> TokenWorkload:
    rng = np.random.default_rng(seed)
    sm = 1.0 / math.sqrt(d_qk)
    q = bf16_bits(rng.standard_normal((T, Hq, d_qk), dtype=np.float32))
    # K and V share the same bytes (V = leading d_v columns), so the codes are
    # N(0,1) at unit scale and read back with both k_scale and v_scale.
    kv = _normal_codes(rng, (S, d_qk))
    sink = _sink_for(rng, Hq, topk, sm, q_scale or 1.0) if with_sink else None
    idx = _distinct_sorted(rng, T, topk, S)
    return TokenWorkload(name, q, kv, idx, sink, sm, d_v, q_scale, k_scale, v_scale)


def block_workload(B: int, seq_len: int, q_len: int, *, seed: int, name: str, Hq=16, Hkv=2,
                   Hidx=4, D=128, Didx=128, topk=64, scales=None, exact_index=False,
                   with_sink=False, extra_pages: int = 0) -> BlockWorkload:
    """B sequences of ``seq_len`` tokens whose last ``q_len`` tokens are queries.

    ``scales``: None (all unit) or ``"uniform"`` (q, k, v, idx_q, idx_k ~ U(0.1, 4)).
    ``exact_index``: additionally draw index-query / index-key codes whose values
    are e4m3-exact integers (|q| <= 64, |k| <= 16) so that every index dot
    product is an integer below 2^17 (stored in ``extra``).
    """
    rng = np.random.default_rng(seed)
    T = B * q_len
    nb = (seq_len + PAGE - 1) // PAGE
    P = B * nb + extra_pages
    q = bf16_bits(rng.standard_normal((T, Hq, D), dtype=np.float32))
    iq = bf16_bits(rng.standard_normal((T, Hidx, Didx), dtype=np.float32))
    # scales are drawn after the caches in the recipe, but the cache codes depend
    # on them; draw them from an independent child stream so the order holds.
    sc_rng = np.random.default_rng([seed, 5])
    sc = None
    if scales == "uniform":
        sc = sc_rng.uniform(0.1, 4.0, size=5)
    k_s = None if sc is None else float(sc[1])
    v_s = None if sc is None else float(sc[2])
    iq_s = None if sc is None else float(sc[3])
    ik_s = None if sc is None else float(sc[4])
    q_s = None if sc is None else float(sc[0])
    kc = _normal_codes(rng, (P, Hkv, PAGE, D), std=1.0 / (k_s or 1.0))
    vc = _normal_codes(rng, (P, Hkv, PAGE, D), std=1.0 / (v_s or 1.0))
    ik = _normal_codes(rng, (P, PAGE, Didx), std=1.0 / (ik_s or 1.0))
    sm = 1.0 / math.sqrt(D)
    sink = _sink_for(rng, Hq, topk * PAGE, sm, q_s or 1.0) if with_sink else None
    perm = rng.permutation(P).astype(np.int32)
    bt = perm[: B * nb].reshape(B, nb)
    cu = (np.arange(B + 1) * q_len).astype(np.int32)
    sl = np.full(B, seq_len, dtype=np.int32)
    extra = {}
    if exact_index:
        extra["idx_q8_exact"], extra["idx_k8_exact"] = exact_index_codes(seed, T, Hidx, Didx, P)
    return BlockWorkload(name, q, iq, kc, vc, ik, bt, cu, sl, q_len, topk, sm, 1.0 / math.sqrt(Didx),
                         q_s, k_s, v_s, iq_s, ik_s, sink, extra)


def exact_index_codes(seed: int, T: int, Hidx: int, Didx: int, P: int, chunk_pages: int = 1024):
    """Exact-mode index codes of a block workload: e4m3-exact integers with
    random signs, |q| <= 64 for the index query ``[T, Hidx, Didx]`` and
    |k| <= 16 for the index-key cache ``[P, PAGE, Didx]``, drawn from the
    child stream ``[seed, 7]`` (so they leave the workload's other draws
    unchanged).  The key cache is drawn in chunks of ``chunk_pages`` pages to
    bound memory."""
    ex_rng = np.random.default_rng([seed, 7])
    qv = ex_rng.choice(E4M3_EXACT_INTS, size=(T, Hidx, Didx)) * ex_rng.choice([-1.0, 1.0], size=(T, Hidx, Didx))
    iq = e4m3_codes(qv.astype(np.float32))
    del qv
    ik = np.empty((P, PAGE, Didx), np.uint8)
    kvals = E4M3_EXACT_INTS[E4M3_EXACT_INTS <= 16]
    for p0 in range(0, P, chunk_pages):
        n = min(chunk_pages, P - p0)
        kv = ex_rng.choice(kvals, size=(n, PAGE, Didx)) * ex_rng.choice([-1.0, 1.0], size=(n, PAGE, Didx))
        ik[p0:p0 + n] = e4m3_codes(kv.astype(np.float32))
    return iq, ik


def workload(n: int, small: bool = False):
    """Workload ``n`` (1..5) at its full size, or a reduced size for quick checks."""
    seed = 1000 + n
    if n == 1:
        return token_workload(64, 16, 4096, 256, seed=seed, name="mla_tiny_64x16_s4096_top256",
                              q_scale=0.5, k_scale=0.25, v_scale=2.0)
    if n == 2:
        L = 1024 if small else 8192
        return block_workload(1, L, L, seed=seed, name=f"gqa_prefill_{L}_h16kv2_top64")
    if n == 3:
        L = 2048 if small else 32768
        return block_workload(1, L, L, seed=seed, name=f"gqa_prefill_{L}_h16kv2_top64_scaled",
                              scales="uniform", exact_index=True)
    if n == 4:
        T, S = (64, 8192) if small else (4096, 65536)
        return token_workload(T, 128, S, 2048, seed=seed, name=f"mla_prefill_{T}x128_s{S}_top2048")
    if n == 5:
        B, L = (8, 16384) if small else (64, 32768)
        return block_workload(B, L, 1, seed=seed, name=f"gqa_decode_b{B}_s{L}_top64")
    raise ValueError(n)
