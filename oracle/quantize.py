"""Per-tensor fp8 quantization (test infrastructure only).

What the pages define
---------------------
* The fp8 tensor stores value / scale and consumers multiply the scale back;
  ``None`` means unit scale and no division at all (sglang PR 30971 digest,
  implementation step 3 and the ``_quant_q_fp8`` code excerpt).
* The quantize kernel converts each element to fp32, multiplies by a single
  ``scale_inv`` and casts to e4m3 (sglang PR 25460 digest, code excerpt of
  ``_fp8_quantize_kernel``); a 2-D row-strided view is formed from the
  leading dimensions (same excerpt, ``_flatten_to_2d``).

Reading taken where the two pages differ: the MiniMax wrapper divides in the
input's dtype while the Triton kernel multiplies in fp32.  The oracle follows
the fp32 multiply by a reciprocal rounded once to fp32 on the host:
``scale_inv = fl32(1 / fl32(scale))``, ``y = e4m3(fl32(fl32(x) * scale_inv))``;
with no scale the multiply is skipped.  This precision is fixed by the page
(fp32), so the oracle computes in fp32 here, not float64.

Pins (tests/test_oracle_quantize.py): exhaustive over all 65536 bf16 and fp16
bit patterns, the oracle equals torch's CPU fp32 multiply followed by torch's
e4m3fn cast wherever that cast is defined (|v| < 464); scale None equals
scale 1.0; power-of-two scales commute exactly with the grid.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import e4m3

BF16 = 0
FP16 = 1


def widen_to_fp32(bits, dtype: int) -> np.ndarray:
    """Exact widening of bf16 / fp16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    if dtype == FP16:
        return b.view(np.float16).astype(np.float32)
    raise ValueError(f"unknown input dtype {dtype}")


def scale_inv_fp32(scale: Optional[float]) -> Optional[np.float32]:
    """fl32(1 / fl32(scale)), computed once (None stays None)."""
    if scale is None:
        return None
    return np.float32(1.0) / np.float32(scale)


def quantize(bits, dtype: int, scale: Optional[float]) -> np.ndarray:
    """Quantize a bf16/fp16 tensor (given as uint16 bit patterns) to e4m3 codes."""
    x = widen_to_fp32(bits, dtype)
    s_inv = scale_inv_fp32(scale)
    if s_inv is None:
        v = x
    else:
        with np.errstate(over="ignore", invalid="ignore"):
            v = (x * s_inv).astype(np.float32)   # one IEEE fp32 multiply
    return e4m3.encode(v)
