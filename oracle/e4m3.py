"""OCP FP8 e4m3fn codec (test infrastructure only; see ``oracle/__init__``).

The pages store every fp8 tensor in this format: the MiniMax q quantizer casts
to ``torch.float8_e4m3fn`` (sglang PR 30971 digest, code excerpt of
``_quant_q_fp8``), the index cache is ``torch.float8_e4m3fn`` (vLLM PR 45892
digest, implementation step 3), and the quantize kernel maps the e4m3 dtype to
Triton's ``float8e4nv`` (sglang PR 25460 digest, code excerpt of
``fp8_quantize``).  The bit layout is the OCP 8-bit floating point
specification's E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
no infinities, a single NaN mantissa pattern (S.1111.111), largest finite
magnitude 448.

Encoding rule (the pages do not print one; this is the reading used
throughout): round to nearest, ties to even, and saturate every finite or
infinite magnitude that rounds above 448 to 448.  NaN encodes to 0x7F with the
input's sign bit.  Negative zero keeps its sign (0x80).

Pins (tests/test_oracle_e4m3.py): decode is checked code-by-code against the
closed form over all 256 codes; encode is checked against torch's CPU
float8_e4m3fn cast (an RNE library routine) for every finite |v| < 464 over
dense sweeps, against a hand table for saturation, and by the round trip
decode(encode(v)) == v on all 254 finite codes.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6      # smallest normal magnitude
_SUBNORMAL_STEP = 2.0 ** -9  # spacing of the subnormal grid


def decode(codes) -> np.ndarray:
    """Decode e4m3fn byte codes to float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = m.astype(np.float64) * _SUBNORMAL_STEP
    nrm = (1.0 + m.astype(np.float64) / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def encode(values) -> np.ndarray:
    """Encode real values (float32 or float64, taken exactly) to e4m3fn codes.

    Round-to-nearest-even on the e4m3 grid, saturating at +-448.
    """
    with np.errstate(invalid="ignore"):          # signalling-NaN inputs widen quietly
        v = np.asarray(values, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint8)
    neg = np.signbit(v)
    nan = np.isnan(v)
    a = np.abs(np.where(nan, 0.0, v))

    # Grid spacing at |v|: 2^-9 below the smallest normal, else 2^(floor(log2|v|) - 3).
    _, ex = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
    floor_log2 = ex.astype(np.float64) - 1.0
    step = np.where(a < _MIN_NORMAL, _SUBNORMAL_STEP, np.exp2(floor_log2 - 3.0))
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(a / step) * step          # np.rint: ties to even
    r = np.where(np.isfinite(a), r, np.inf)
    r = np.minimum(r, E4M3_MAX)                 # saturation (also for +-inf)

    # Magnitude -> code.
    is_sub = r < _MIN_NORMAL
    m_sub = np.rint(r / _SUBNORMAL_STEP).astype(np.int64)          # 0..7
    _, rex = np.frexp(np.where(is_sub, 1.0, r))
    e_unb = rex.astype(np.int64) - 1                                # floor(log2 r)
    mant = np.rint(np.where(is_sub, 0.0, r / np.exp2(e_unb.astype(np.float64)) * 8.0 - 8.0))
    code_nrm = ((e_unb + 7) << 3) | mant.astype(np.int64)
    mag_code = np.where(is_sub, m_sub, code_nrm)
    mag_code = np.where(nan, 0x7F, mag_code)
    out[...] = (mag_code | np.where(neg, 0x80, 0)).astype(np.uint8)
    return out


def decode_table() -> np.ndarray:
    """Float64 value of every code 0..255 (NaN for the two NaN codes)."""
    return decode(np.arange(256, dtype=np.uint8))
