"""Element codecs of the oracle (test infrastructure only; see package header).

Formats and where the pages name them:

* bfloat16 -- the activation and output type ("Low-Latency Mode API",
  Parameters: ``x`` is bfloat16; Return Values: ``combined_x`` is bfloat16).
* int8 with a float32 per-token scale -- ``use_fp8`` on the NPU
  ("Low-Latency Mode API", Parameters, ``use_fp8``).
* float8_e4m3fn -- MXFP8 data ("Low-Latency Mode API", ``use_ue8m0``) and
  the per-128-channel FP8 path ("DeepEP FP8 Dispatch and Combine
  Operations", "The Dispatch Stage").
* float4_e2m1fn_x2 -- MXFP4 data, two codes per byte ("Low-Latency Mode
  API", ``use_mxfp4``).
* float8_e8m0fnu -- the power-of-two block scale of both MX formats (same
  rows).

The pages name the formats but do not define them; the definitions used here
are the public OCP ones (e4m3fn: bias 7, three mantissa bits, no infinity,
S.1111.111 is NaN, largest finite 448; e2m1: bias 1, one mantissa bit,
magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; e8m0: byte b is 2**(b-127), 0xFF is
NaN).

Rounding is done the slow, obvious way: list every finite value of the target
format, find the two neighbours of the input, take the nearer one, and on a
tie take the code whose least significant bit is zero (round half to even).
All distances are computed in float64, where they are exact for these inputs.

Parity: pinned.  ``f32_to_bf16_bits`` and ``e4m3_encode`` are pinned against
torch's CPU casts (a library routine) over every bfloat16 pattern and over
all midpoints; ``e2m1_encode`` against a hand-written midpoint table from the
OCP value list; the decoders against exhaustive closed forms.  See
``tests/test_oracle_codecs.py``.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 <-> float32
# ---------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of a float32, so widening is a 16-bit shift
    (exact for every pattern, NaN payloads included)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _bf16_value(bits_u32: np.ndarray) -> np.ndarray:
    """float64 value of bfloat16 patterns given as uint32 (finite or inf)."""
    return (bits_u32.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16, ties to even; NaN -> quiet NaN.

    The two candidates are the bfloat16 patterns just below and just above
    |x| in magnitude (truncation, and truncation plus one unit).  For the
    tie-breaking and overflow rule of IEEE round-to-nearest-even, the pattern
    above the largest finite value (0x7F80, infinity) counts as 2**128.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = (u >> np.uint32(16)) & np.uint32(0x8000)
    mag = u & np.uint32(0x7FFFFFFF)
    lo = mag >> np.uint32(16)                      # truncated magnitude pattern
    hi = lo + np.uint32(1)
    xv = mag.view(np.float32).astype(np.float64)
    vlo = _bf16_value(lo)
    vhi = np.where(hi == 0x7F80, 2.0 ** 128, _bf16_value(np.minimum(hi, 0x7F80)))
    # infinite inputs give inf - inf here; they are handled by `is_inf` below
    with np.errstate(invalid="ignore"):
        dlo = xv - vlo
        dhi = vhi - xv
    take_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & np.uint32(1)) == 1))
    take_hi &= mag != (lo << np.uint32(16))         # exact values stay put
    res = np.where(take_hi, hi, lo)
    is_inf = mag == 0x7F800000
    res = np.where(is_inf, np.uint32(0x7F80), res)
    is_nan = mag > 0x7F800000
    res = np.where(is_nan, np.uint32(0x7FC0), res)
    return (res | sign).astype(np.uint16)


# ---------------------------------------------------------------------------
# generic nearest-value rounding onto a small format
# ---------------------------------------------------------------------------


def _round_to_table(mag: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Index of the entry of ascending ``values`` nearest to each ``mag``
    (float64, 0 <= mag <= values[-1]); ties go to the even index.  For the
    formats here the index is the code, so "even index" is "even code"."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(values, mag, side="left")
    hi = np.clip(hi, 0, len(values) - 1)
    lo = np.clip(hi - 1, 0, len(values) - 1)
    dlo = mag - values[lo]
    dhi = values[hi] - mag
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


# ---------------------------------------------------------------------------
# OCP float8 e4m3fn
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn byte: exponent field E (4 bits), mantissa M (3
    bits), bias 7.  E == 0 is subnormal, M/8 * 2**-6; otherwise
    (1 + M/8) * 2**(E-7).  0x7F and 0xFF are NaN.  Returned as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x80) != 0, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


E4M3_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0..0x7E ascending


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values already clamped to [-448, 448] to e4m3fn, round
    half to even, keeping the sign bit (so -0 and tiny negatives give 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.abs(v.astype(np.float64)) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode expects finite input clamped to +-448")
    sign = np.signbit(v)
    code = _round_to_table(np.abs(v.astype(np.float64)), E4M3_POS_VALUES).astype(np.uint8)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)


# ---------------------------------------------------------------------------
# OCP float4 e2m1
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_POS_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each 4-bit e2m1 code (bit 3 is the sign); float64."""
    c = np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)
    mag = E2M1_POS_VALUES[c & 0x7]
    return np.where((c & 0x8) != 0, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values already clamped to [-6, 6] to e2m1 (one code per
    uint8, low nibble), round half to even, keeping the sign bit."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(np.abs(v.astype(np.float64)) > E2M1_MAX) or np.any(np.isnan(v)):
        raise ValueError("e2m1_encode expects finite input clamped to +-6")
    sign = np.signbit(v)
    code = _round_to_table(np.abs(v.astype(np.float64)), E2M1_POS_VALUES).astype(np.uint8)
    return np.where(sign, code | np.uint8(0x8), code).astype(np.uint8)


def pack_e2m1_pairs(codes: np.ndarray) -> np.ndarray:
    """Two e2m1 codes per byte along the last axis: element 2i in the low
    nibble, element 2i+1 in the high nibble (the pages do not fix the order;
    this is the reading taken)."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("odd number of e2m1 codes")
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_e2m1_pairs(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# e8m0 (power-of-two scale byte)
# ---------------------------------------------------------------------------


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """Byte b is 2**(b - 127); 0xFF is NaN.  float64 (exact)."""
    bi = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(bi == 0xFF, np.nan, np.exp2(bi - 127.0))
