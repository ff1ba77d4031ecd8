"""Paged fp8 KV-cache store (test infrastructure only; see ``oracle/__init__``).

What the pages define
---------------------
* The KV pools hold fp8 values as value / scale, with ``None`` meaning unit
  scale and no division at all: the MiniMax pool's K/V, index-K and fused
  K/V/index setters take an Optional scale defaulting to None (sglang PR 30971
  digest, implementation step 4), and the q quantizer states the same storage
  convention as the pool (same digest, ``_quant_q_fp8`` code excerpt).
* The MLA prefill hook writes the KV cache directly in fp8, packing the latent
  part (``kv_a``) and the rope part (``k_pe``) of each token into one cache
  row (sglang PR 25460 digest, implementation step 2, ``mla_kv_pack_quantize_fp8``).
* Each element is quantized as the quantize step does it: widen to fp32,
  multiply by the fp32 reciprocal of the scale, round to e4m3 (same digest,
  ``_fp8_quantize_kernel`` excerpt).  ``quantize.quantize`` is that step.

Readings taken where the pages are silent
-----------------------------------------
* Slot mapping: token n goes to slot s = slot_mapping[n], i.e. page
  s // page_size at in-page offset s % page_size (the usual paged layout).
  A negative slot (a padding token) or a slot at or beyond
  num_pages * page_size writes nothing.  A slot is named at most once per call.
* Cache layout ``[num_pages, num_heads, page_size, row]`` with
  row = dim (+ dim2): the block-mode K/V caches ``[pages, Hkv, 128, 128]``,
  the single-head index-K cache (num_heads = 1) and the flat MLA KV array
  ``[S, 576]`` (num_heads = 1, page_size = 1) are all this shape.
* With a second source (dim2 > 0) its codes fill columns dim .. dim+dim2-1 of
  the same row, quantized with the same scale.

Pins (tests/test_oracle_cache_store.py): a hand-placed byte table for a tiny
layout (slot -> page, offset, head axis, both sources, skipped slots) whose
codes come from the OCP e4m3 bit layout; read-back invariants (every stored
row equals the quantized source row, every other byte is unchanged); the
round trip decode(code) * scale == x for e4m3-exact values and power-of-two
scales.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import quantize as _q


def cache_store(cache: np.ndarray, x_bits: np.ndarray, dtype: int, slot_mapping: np.ndarray,
                scale: Optional[float], x2_bits: Optional[np.ndarray] = None) -> np.ndarray:
    """Return a copy of ``cache`` [pages, H, page_size, row] with the tokens stored.

    x_bits:  uint16 bf16/fp16 bit patterns [N, H, dim].
    x2_bits: optional second source [N, H, dim2] placed after x in each row.
    slot_mapping: integer [N].
    """
    out = np.array(cache, dtype=np.uint8, copy=True)
    pages, heads, page_size, row = out.shape
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n_tok, xh, dim = x_bits.shape
    assert xh == heads, "source head count must match the cache"
    codes = _q.quantize(x_bits, dtype, scale)
    codes2 = None
    dim2 = 0
    if x2_bits is not None:
        x2_bits = np.asarray(x2_bits, dtype=np.uint16)
        assert x2_bits.shape[:2] == (n_tok, heads)
        dim2 = x2_bits.shape[2]
        codes2 = _q.quantize(x2_bits, dtype, scale)
    assert dim + dim2 == row, "cache row must hold dim + dim2 bytes"
    n_slots = pages * page_size
    for n in range(n_tok):
        s = int(slot_mapping[n])
        if s < 0 or s >= n_slots:
            continue
        page, off = divmod(s, page_size)
        out[page, :, off, :dim] = codes[n]
        if codes2 is not None:
            out[page, :, off, dim:] = codes2[n]
    return out
