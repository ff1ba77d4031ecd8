"""Rotary position embedding fused with e4m3 quantization (test infrastructure only;
see ``oracle/__init__``).

What the pages define
---------------------
* The MLA prefill hook applies RoPE to the rope part of Q and K and quantizes
  both parts to e4m3 in one fused producer, writing each head's no-rope part
  followed by its rope part as one contiguous fp8 row, so the attention kernel
  needs no concat or cast (sglang PR 25460 digest, implementation step 2 and
  the ``_fused_rope_fp8_quantize`` excerpt).  Its inputs are the no-rope and
  rope parts, a ``cos_sin_cache`` indexed by token position, the positions, an
  ``is_neox`` switch and a per-tensor quantization scale.  A rope part shared
  by all heads (K's single rope head) is broadcast to every head (same
  excerpt: "RoPE depends only on the position").
* Quantization is the quantize step's: multiply by the fp32 reciprocal of
  the scale, round to e4m3 (same digest, ``_fp8_quantize_kernel`` excerpt);
  None skips the multiply.

RoPE itself is the rotary embedding of Su et al. (RoFormer, 2021): the rope
dims form pairs, and pair i at position p is rotated by the angle p * theta_i,
    (a, b) -> (a cos - b sin,  b cos + a sin).

Readings taken where the pages are silent
-----------------------------------------
* ``cos_sin_cache`` is fp32 ``[max_position, rope_dim]``: row p holds the rope_dim/2
  cosines of pair angles at position p, then the rope_dim/2 sines.
* Pairing: ``is_neox`` pairs dim i with dim i + rope_dim/2 (rotate-half);
  otherwise dims 2i and 2i+1 are paired (interleaved).  Pair i uses column i
  of the cosine and sine halves in both layouts.
* Precision: the rotation is evaluated in fp32 with every product rounded
  separately: fl32(fl32(a cos) - fl32(b sin)) and fl32(fl32(b cos) + fl32(a sin)),
  then fl32(* scale_inv), then e4m3.  The pages fix no precision here, so the
  quantized codes are decided in the kernel's fp32 arithmetic, which both
  sides follow operation by operation.
* A position outside [0, max_position) writes NaN codes (0x7F) over the rope
  part of that token's rows, so the error stays visible downstream; the
  no-rope part is quantized as usual.

Pins (tests/test_oracle_rope.py): position 0 (cos 1, sin 0) reduces to plain
quantization; quarter and half turns given exactly in the cache reduce to a
hand-written permutation and negation of the inputs (pairing convention and
signs); the fp32 rotation agrees with complex128 multiplication
(a + ib)(cos + i sin) within the fp32 rounding bound; a broadcast rope head
rotates identically for every head; out-of-range positions give 0x7F.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import e4m3 as _e
from . import quantize as _q

NAN_CODE = 0x7F


def rope_fp32(x_pe: np.ndarray, cos_sin_cache: np.ndarray, positions: np.ndarray,
              is_neox: bool) -> np.ndarray:
    """fp32 rotation of x_pe [T, H, R] (float32) at positions [T] (valid ones only)."""
    x = np.asarray(x_pe, dtype=np.float32)
    R = x.shape[-1]
    half = R // 2
    cs = np.asarray(cos_sin_cache, dtype=np.float32)[np.asarray(positions, dtype=np.int64)]
    c = cs[:, None, :half]
    s = cs[:, None, half:]
    if is_neox:
        a, b = x[..., :half], x[..., half:]
    else:
        a, b = x[..., 0::2], x[..., 1::2]
    ra = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    rb = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    out = np.empty_like(x)
    if is_neox:
        out[..., :half], out[..., half:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out


def rope_quantize(x_nope_bits: Optional[np.ndarray], x_pe_bits: np.ndarray, dtype: int,
                  cos_sin_cache: np.ndarray, positions: np.ndarray, is_neox: bool,
                  scale: Optional[float]) -> np.ndarray:
    """e4m3 codes [T, H, nope + rope]: quantize(x_nope) ++ quantize(rope(x_pe)).

    x_nope_bits: uint16 [T, H, nope] or None; x_pe_bits: uint16 [T, H or 1, R].
    """
    pe = _q.widen_to_fp32(x_pe_bits, dtype)
    T, hp, R = pe.shape
    H = hp if x_nope_bits is None else np.asarray(x_nope_bits).shape[1]
    pe = np.broadcast_to(pe, (T, H, R))
    pos = np.asarray(positions, dtype=np.int64)
    valid = (pos >= 0) & (pos < cos_sin_cache.shape[0])
    rot = np.zeros((T, H, R), dtype=np.float32)
    if valid.any():
        rot[valid] = rope_fp32(pe[valid], cos_sin_cache, pos[valid], is_neox)
    s_inv = _q.scale_inv_fp32(scale)
    if s_inv is not None:
        with np.errstate(over="ignore", invalid="ignore"):
            rot = (rot * s_inv).astype(np.float32)
    codes_pe = _e.encode(rot)
    codes_pe[~valid] = NAN_CODE
    if x_nope_bits is None:
        return codes_pe
    codes_nope = _q.quantize(x_nope_bits, dtype, scale)
    return np.concatenate([codes_nope, codes_pe], axis=-1)
