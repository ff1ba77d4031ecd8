"""Plain CPU oracle for FP8-e4m3 top-k sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding in ``fp8_top_sparse_amd``) imports, links or calls this
package.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant generator with the GPU path.

Every function here is a slow, obviously-correct restatement of what the
source pages define, evaluated in float64 on dequantized fp8 inputs (the
pages' "dequantized reference" test strategy), except where the pages fix a
narrower precision (the fp32 multiply inside quantization).

Modules
-------
e4m3       OCP e4m3fn decode / round-to-nearest-even encode with saturation.
quantize   per-tensor fp8 quantization ("stored value = x / scale").
indexer    lightning-indexer block scores and ascending top-k block ids.
attention  sparse attention forward (token mode and block mode).
cache_store  quantize new K / V / index-K rows into a paged fp8 cache.
rope       rotary position embedding fused with e4m3 quantization.
qknorm     per-head RMS norm + RoPE + e4m3 quantization (+ paged store) of index q / k.

Pins: every function is checked by ``tests/test_oracle_*.py`` against closed
forms, exhaustive enumeration, brute force and library routines; the pin for
each function is listed in its docstring.
"""

from . import e4m3, quantize, indexer, attention, cache_store, rope, qknorm  # noqa: F401

__all__ = ["e4m3", "quantize", "indexer", "attention", "cache_store", "rope", "qknorm"]
