"""Per-row quantisation of the oracle (test infrastructure only).

Every token row is quantised once, then copied to each routed row.  The seven
modes and the passages they follow:

* ``none``       -- bf16 passes through ("Low-Latency Mode API", Return
  Values: BF16 when ``use_fp8`` is off).
* ``int8_token`` -- per-token dynamic int8 with a float32 scale (same page,
  Parameters, ``use_fp8``; Return Values: int8 data plus one float32 per
  token).  Scale = amax/127, round half to even, clamp to +-127.
* ``fp8_b128``   -- e4m3 codes with one float32 scale per 128-channel block
  ("DeepEP FP8 Dispatch and Combine Operations", "The Dispatch Stage": the
  hidden dimension is cut into 128-element blocks, each with its own amax
  and scale; "The FP8 Combine Operation": the stored inverse scale multiplies
  the codes back).  The page prints the multiplier as 127/amax; for e4m3 the
  largest code is 448, so the oracle uses 448.
* ``fp8_b128_pow2`` -- as ``fp8_b128`` with every scale rounded to a power
  of two ("DeepEP FP8 Dispatch and Combine Operations", Advanced
  Configuration Options: ``round_scale``; "Low-Latency Mode API",
  Parameters: ``round_scale``).  The page says "nearest"; rounding a scale
  down would push the block's largest element past 448, so the reading
  taken is: round the computed scale UP to the next power of two.
* ``fp8_b128_ue8m0`` -- the same codes and power-of-two scales, each scale
  stored as one e8m0 byte instead of a float32 (same page and section:
  ``use_ue8m0`` packs the scales into 8 bits); byte g of a row's scales is
  128-channel block g, so four consecutive blocks share one int32.
* ``mxfp8``      -- e4m3 codes plus one e8m0 scale per 32-element block
  ("Low-Latency Mode API", ``use_ue8m0``).
* ``mxfp4``      -- e2m1 codes, two per byte, plus one e8m0 scale per
  32-element block ("Low-Latency Mode API", ``use_mxfp4``).

Arithmetic for the scaled modes (the pages give the scale, not the order of
operations; this is the reading taken): with ``qmax`` the largest code
(127 or 448), the multiplier ``m = fl32(qmax / amax)`` scales the elements
and the stored scale is ``s = fl32(amax / qmax)`` -- two separate float32
divisions, each rounded once.  Each element is ``fl32(x * m)``, clamped to
+-qmax and rounded to the code.  If ``amax`` is zero or ``m`` is not finite
the block stores scale 0 and all codes 0 (the pages are silent on this case).

Power-of-two scale (``fp8_b128_pow2`` / ``fp8_b128_ue8m0``): with
``s0 = fl32(amax / 448)`` (the ``fp8_b128`` scale) and ``e = ceil(log2 s0)``
read off the float32 bits of s0, the scale is ``2**e`` and the multiplier
``2**-e``; both are exact, so each element is ``fl32(x * 2**-e)`` (exact
unless it falls below float32's normal range), clamped to +-448 and rounded
to e4m3.  A block with amax zero, or with ``e < -127`` (its multiplier would
overflow float32, the same condition under which ``fp8_b128`` zeroes a
block), stores scale 0 (byte 0) and zero codes.  The e8m0 byte is ``e + 127``.

MX scale rule (the pages give only the block size, 32 elements, and the scale
format; this is the OCP MX rule): with ``e = floor(log2(amax))`` and ``emax`` the
exponent of the element format's largest value (8 for e4m3, whose largest is
1.75 * 2**8; 2 for e2m1, whose largest is 1.5 * 2**2), the shared exponent is
``clamp(e - emax, -127, 127)`` (-127 when amax is zero) and the stored byte
is that plus 127.  Elements are ``fl32(x * 2**-exp)``, clamped to the
element format's largest value, then rounded.

Parity: ``fp8_b128_pow2``/``ue8m0`` pinned by the properties "scale is the
smallest power of two >= s0", |code value| <= 448, the per-element error
bound, reduction to ``fp8_b128`` when s0 is itself a power of two, and a hand
example.  ``int8``/``fp8_b128`` pinned by the properties |q| <= qmax, the amax
element mapping to +-qmax and the per-element error bound; the MX scale byte
pinned by recomputation with ``math.frexp``; all element rounding is in
``codecs`` (pinned there).  The MX rule itself is pinned only by the OCP MX
specification, which is not among the pages: that part is "parity unpinned"
with respect to the pages.
"""

from __future__ import annotations

import numpy as np

from . import codecs

INT8_QMAX = np.float32(127.0)
E4M3_QMAX = np.float32(448.0)

# bytes of data and of scales per row, by mode (hidden size H)


def row_bytes(mode: str, hidden: int) -> tuple[int, int]:
    """(data bytes, scale bytes) of one packed row -- the receive layout of
    "Low-Latency Mode API", Return Values, with the FP8 per-128 scales as in
    "DeepEP FP8 Dispatch and Combine Operations"."""
    if mode == "none":
        return 2 * hidden, 0
    if mode == "int8_token":
        return hidden, 4
    if mode in ("fp8_b128", "fp8_b128_pow2"):
        return hidden, 4 * (hidden // 128)
    if mode == "fp8_b128_ue8m0":
        return hidden, hidden // 128
    if mode == "mxfp8":
        return hidden, hidden // 32
    if mode == "mxfp4":
        return hidden // 2, hidden // 32
    raise ValueError(f"unknown quant mode {mode!r}")


def _amax(x_f32: np.ndarray) -> np.float32:
    """Largest magnitude of a block, exact in float32."""
    return np.float32(np.max(np.abs(x_f32))) if x_f32.size else np.float32(0.0)


def _scaled_block(x_f32: np.ndarray, qmax: np.float32):
    """Multiplier, stored scale and the scaled, clamped elements of one block
    (see the module header)."""
    amax = _amax(x_f32)
    with np.errstate(divide="ignore", over="ignore"):
        m = np.float32(qmax / amax) if amax != 0 else np.float32(np.inf)
    if amax == 0 or not np.isfinite(m):
        return np.float32(0.0), np.zeros_like(x_f32), True
    s = np.float32(amax / qmax)
    v = (x_f32 * m).astype(np.float32)
    v = np.clip(v, -qmax, qmax).astype(np.float32)
    return s, v, False


def quant_int8_token(x_bits: np.ndarray):
    """One bf16 row -> (int8 codes [H], float32 scale)."""
    x = codecs.bf16_bits_to_f32(x_bits)
    s, v, zero = _scaled_block(x, INT8_QMAX)
    if zero:
        return np.zeros(x.shape, np.int8), np.float32(0.0)
    q = np.rint(v)                       # round half to even
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def quant_fp8_b128(x_bits: np.ndarray):
    """One bf16 row -> (e4m3 codes [H] uint8, float32 scales [H/128])."""
    x = codecs.bf16_bits_to_f32(x_bits)
    H = x.shape[0]
    codes = np.empty(H, np.uint8)
    scales = np.empty(H // 128, np.float32)
    for g in range(H // 128):
        blk = x[g * 128:(g + 1) * 128]
        s, v, zero = _scaled_block(blk, E4M3_QMAX)
        scales[g] = s
        codes[g * 128:(g + 1) * 128] = 0 if zero else codecs.e4m3_encode(v)
    return codes, scales


def ceil_log2(s: np.float32) -> int:
    """ceil(log2 s) of a positive finite float32, from its bit pattern: the
    exponent of the leading one, plus one unless s is a power of two."""
    b = int(np.float32(s).view(np.uint32)) & 0x7FFFFFFF
    if b == 0 or b >= 0x7F800000:
        raise ValueError("ceil_log2 needs a positive finite value")
    ef, mant = b >> 23, b & 0x7FFFFF
    if ef == 0:                            # subnormal: s = mant * 2**-149
        lead = mant.bit_length() - 1
        return lead - 149 + (0 if mant == 1 << lead else 1)
    return ef - 127 + (0 if mant == 0 else 1)


def quant_fp8_b128_pow2(x_bits: np.ndarray):
    """One bf16 row -> (e4m3 codes [H] uint8, exponents e [H/128] (int, the
    scale is 2**e), zero flags [H/128])."""
    x = codecs.bf16_bits_to_f32(x_bits)
    H = x.shape[0]
    codes = np.zeros(H, np.uint8)
    exps = np.zeros(H // 128, np.int64)
    zero = np.zeros(H // 128, bool)
    for g in range(H // 128):
        blk = x[g * 128:(g + 1) * 128]
        amax = _amax(blk)
        if amax == 0:
            zero[g] = True
            continue
        e = ceil_log2(np.float32(amax / E4M3_QMAX))
        if e < -127:
            zero[g] = True
            continue
        exps[g] = e
        v = (blk.astype(np.float64) * 2.0 ** -e).astype(np.float32)    # one rounding
        v = np.clip(v, -E4M3_QMAX, E4M3_QMAX).astype(np.float32)
        codes[g * 128:(g + 1) * 128] = codecs.e4m3_encode(v)
    return codes, exps, zero


def mx_shared_exponent(amax: np.float32, emax: int) -> int:
    """Shared exponent of an MX block: clamp(floor(log2 amax) - emax, -127,
    127), or -127 for amax == 0.  floor(log2 amax) is read off the float32
    bit pattern: the biased exponent field, or for a subnormal amax the
    position of its leading one."""
    a = int(np.float32(amax).view(np.uint32)) & 0x7FFFFFFF
    if a == 0:
        return -127
    ef = a >> 23
    if ef == 0:                            # subnormal: value = mant * 2**-149
        e = (a.bit_length() - 1) - 149
    else:
        e = ef - 127
    return max(-127, min(127, e - emax))


def _quant_mx(x_bits: np.ndarray, emax: int, vmax: float, encode):
    return _quant_mx_values(codecs.bf16_bits_to_f32(x_bits), emax, vmax, encode)


def _quant_mx_values(x: np.ndarray, emax: int, vmax: float, encode):
    """The MX rule on a float32 row (length a multiple of 32)."""
    x = np.asarray(x, dtype=np.float32)
    H = x.shape[0]
    codes = np.empty(H, np.uint8)
    scale_bytes = np.empty(H // 32, np.uint8)
    for g in range(H // 32):
        blk = x[g * 32:(g + 1) * 32]
        se = mx_shared_exponent(_amax(blk), emax)
        scale_bytes[g] = se + 127
        # x * 2**-se: exact in float64, then one rounding to float32
        v = (blk.astype(np.float64) * (2.0 ** -se)).astype(np.float32)
        v = np.clip(v, np.float32(-vmax), np.float32(vmax)).astype(np.float32)
        codes[g * 32:(g + 1) * 32] = encode(v)
    return codes, scale_bytes


def quant_mxfp8(x_bits: np.ndarray):
    """One bf16 row -> (e4m3 codes [H] uint8, e8m0 scale bytes [H/32])."""
    return _quant_mx(x_bits, 8, codecs.E4M3_MAX, codecs.e4m3_encode)


def quant_mxfp8_f32(x_f32: np.ndarray):
    """One float32 row -> (e4m3 codes uint8, e8m0 scale bytes per 32): the
    MXFP8 rule of ``quant_mxfp8`` applied to float32 values (the requant of
    an activation that is not bf16)."""
    if not np.all(np.isfinite(np.asarray(x_f32, np.float32))):
        raise ValueError("MX quantisation needs finite input")
    return _quant_mx_values(x_f32, 8, codecs.E4M3_MAX, codecs.e4m3_encode)


def quant_mxfp4(x_bits: np.ndarray):
    """One bf16 row -> (packed e2m1 bytes [H/2], e8m0 scale bytes [H/32])."""
    codes, sb = _quant_mx(x_bits, 2, codecs.E2M1_MAX, codecs.e2m1_encode)
    return codecs.pack_e2m1_pairs(codes), sb


def quantize_row(mode: str, x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """One bf16 row (uint16 patterns) -> (data bytes, scale bytes) exactly as
    they are laid out in a receive row (little-endian scalars)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if mode == "none":
        return x_bits.view(np.uint8).copy(), np.zeros(0, np.uint8)
    if mode == "int8_token":
        q, s = quant_int8_token(x_bits)
        return q.view(np.uint8), np.array([s], np.float32).view(np.uint8)
    if mode == "fp8_b128":
        q, s = quant_fp8_b128(x_bits)
        return q, s.astype("<f4").view(np.uint8)
    if mode in ("fp8_b128_pow2", "fp8_b128_ue8m0"):
        q, e, zero = quant_fp8_b128_pow2(x_bits)
        if mode == "fp8_b128_ue8m0":
            return q, np.where(zero, 0, e + 127).astype(np.uint8)
        s = np.where(zero, 0.0, np.exp2(e.astype(np.float64))).astype("<f4")   # exact powers of two
        return q, s.view(np.uint8)
    if mode == "mxfp8":
        return quant_mxfp8(x_bits)
    if mode == "mxfp4":
        return quant_mxfp4(x_bits)
    raise ValueError(f"unknown quant mode {mode!r}")


def dequantize_row(mode: str, data: np.ndarray, scales: np.ndarray, hidden: int) -> np.ndarray:
    """Row bytes -> float32 values, one rounding per element.

    ``none``: the bf16 value.  ``int8_token`` and ``fp8_b128``: fl32(code *
    scale) ("DeepEP FP8 Dispatch and Combine Operations", "The FP8 Combine
    Operation": codes times the stored inverse scale, through float32);
    ``fp8_b128_pow2`` likewise.  ``fp8_b128_ue8m0`` and MX:
    code value times 2**(b-127), formed exactly in float64 and rounded once to
    float32 (the same number a float32 multiply by the exact power of two
    gives).
    """
    data = np.asarray(data, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if mode == "none":
        return codecs.bf16_bits_to_f32(data.view(np.uint16))
    if mode == "int8_token":
        s = scales.view(np.float32)[0]
        return (data.view(np.int8).astype(np.float32) * s).astype(np.float32)
    if mode in ("fp8_b128", "fp8_b128_pow2"):
        s = np.repeat(scales.view("<f4").astype(np.float32), 128)
        val = codecs.e4m3_decode(data).astype(np.float32)     # exact
        # a power-of-two scale can take a code past float32's range: +-inf (IEEE)
        with np.errstate(over="ignore"):
            return (val * s).astype(np.float32)
    if mode == "fp8_b128_ue8m0":
        sc = np.repeat(codecs.e8m0_decode(scales), 128)
        with np.errstate(over="ignore", invalid="ignore"):
            return (codecs.e4m3_decode(data) * sc).astype(np.float32)
    if mode in ("mxfp8", "mxfp4"):
        if mode == "mxfp8":
            val = codecs.e4m3_decode(data)
        else:
            val = codecs.e2m1_decode(codecs.unpack_e2m1_pairs(data))
        sc = np.repeat(codecs.e8m0_decode(scales), 32)
        with np.errstate(over="ignore", invalid="ignore"):
            return (val * sc).astype(np.float32)
    raise ValueError(f"unknown quant mode {mode!r}")
