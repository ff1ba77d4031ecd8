"""Per-head RMS normalisation, RoPE and e4m3 quantization of index queries and
keys, with an optional store of the codes into a paged fp8 cache (test
infrastructure only; see ``oracle/__init__``).

What the pages define
---------------------
* With an e4m3 index cache, the fused qk-norm + RoPE + KV-insert kernel of the
  MiniMax model writes the index query directly in fp8: its dtype follows the
  index cache's (vLLM PR 45892 digest, implementation step 3), and the fp8
  index path is tested against the bf16 one (same digest, step 5).
* RoPE and the fp32 quantization are the MLA producer's (``oracle.rope``); the
  paged store uses the KV pools' slot layout (``oracle.cache_store``).

Readings taken where the pages are silent
-----------------------------------------
* qk-norm is RMS normalisation over each head's head_dim values with a learned
  weight w[head_dim]:  y_i = x_i * r * w_i,  r = 1 / sqrt(mean_i(x_i^2) + eps).
* Order: normalise, then rotate the last rope_dim dims of the normalised row
  (pairing, cos/sin layout and invalid positions as in ``oracle.rope``), then
  quantize every dim; the first head_dim - rope_dim dims are not rotated.  This
  is the row layout of the MLA producer (no-rope part, then rope part).
* Precision.  The sum of squares is the exact sum of the squares (each square
  of a bf16 or fp16 value is exact in fp64) rounded once to fp64; then
  mean = fl64(ss / head_dim), r = fl32(fl64(1 / fl64(sqrt(fl64(mean + eps))))),
  y_i = fl32(fl32(x_i * r) * w_i).  The rotation and the scale follow in fp32
  as in ``oracle.rope``.  The pages fix no precision; fp64 for the reduction
  makes the normaliser, and so every code, independent of the order in which
  a kernel adds the squares whenever that sum is exact in fp64 (for bf16
  inputs: whenever a row's nonzero magnitudes span less than 2^15).
* Outputs: the codes ``[T, H, head_dim]``, and/or the same rows stored into a
  cache ``[num_pages, H, page_size, head_dim]`` at slot_mapping[t] (negative or
  out-of-range slots write nothing), as ``oracle.cache_store`` places rows.

Pins (tests/test_oracle_qknorm.py): rows of equal magnitude normalise to
exactly +-w (hand-computed codes); a power-of-two rescaling of the input
leaves the codes unchanged; eps enters as a closed form (a row of zeros, and a
row where eps fixes r); the normalised values agree with the plain float64
formula within fp32 rounding; quarter turns rotate only the last rope_dim dims
(hand permutation); invalid positions give 0x7F over the rope dims only; a
hand-placed slot table for the cache store.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import e4m3 as _e
from . import quantize as _q
from .rope import NAN_CODE, rope_fp32


def rms_norm_fp32(x_bits: np.ndarray, dtype: int, weight: np.ndarray, eps: float) -> np.ndarray:
    """fp32 y [T, H, D] = x * r * w with r decided in fp64 from the exact sum of squares."""
    x = _q.widen_to_fp32(x_bits, dtype)
    T, H, D = x.shape
    w = np.asarray(weight, dtype=np.float32)
    eps64 = float(np.float32(eps))
    r = np.empty((T, H), dtype=np.float32)
    x64 = x.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        for t in range(T):
            for h in range(H):
                row = x64[t, h]
                if not np.all(np.isfinite(row)):
                    ss = float(np.sum(row * row))          # inf or NaN, whatever the order
                else:
                    ss = math.fsum((row * row).tolist())   # exact sum, rounded once
                den = math.sqrt(ss / D + eps64)     # eps >= 0: the argument is >= 0, inf or NaN
                r64 = float("inf") if den == 0.0 else 1.0 / den
                r[t, h] = np.float32(r64)
        y = (x * r[:, :, None]).astype(np.float32)
        y = (y * w[None, None, :]).astype(np.float32)
    return y


def qknorm_rope_quantize(x_bits: np.ndarray, dtype: int, weight: np.ndarray, eps: float,
                         cos_sin_cache: np.ndarray, positions: np.ndarray, rope_dim: int,
                         is_neox: bool, scale: Optional[float]) -> np.ndarray:
    """e4m3 codes [T, H, D] of quantize(rope_last_R(rms_norm(x)))."""
    y = rms_norm_fp32(x_bits, dtype, weight, eps)
    T, H, D = y.shape
    R = int(rope_dim)
    pos = np.asarray(positions, dtype=np.int64)
    valid = (pos >= 0) & (pos < cos_sin_cache.shape[0])
    out = y.copy()
    if R > 0 and valid.any():
        out[valid, :, D - R:] = rope_fp32(y[valid][:, :, D - R:], cos_sin_cache, pos[valid], is_neox)
    s_inv = _q.scale_inv_fp32(scale)
    if s_inv is not None:
        with np.errstate(over="ignore", invalid="ignore"):
            out = (out * s_inv).astype(np.float32)
    codes = _e.encode(out)
    if R > 0:
        codes[~valid, :, D - R:] = NAN_CODE
    return codes


def store_rows(cache: np.ndarray, codes: np.ndarray, slot_mapping: np.ndarray) -> np.ndarray:
    """Place codes [T, H, D] into cache [pages, H, page_size, D] by slot (in place; returned)."""
    pages, H, page_size, D = cache.shape
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0 or s >= pages * page_size:
            continue
        cache[s // page_size, :, s % page_size, :] = codes[t]
    return cache
