"""Pins of the oracle's per-row quantisation.

* int8 and per-128 e4m3: the code bound |q| <= qmax, the amax element mapping
  to +-qmax, the per-element error bound of round-to-nearest, and small rows
  whose codes are worked out by hand (ties to even included);
* MX: the shared-exponent byte recomputed independently with ``math.frexp``
  in float64; the scaled amax lands in [2**emax, 2**(emax+1)) before the
  clamp; codes never exceed the element format's maximum;
* zero and tiny blocks store scale 0 / byte 0 and zero codes.
"""

import math

import numpy as np
import pytest

from combine_topk_idx_amd.workloads import bf16_from_f32
from oracle import codecs, quant


def _row(seed, H, scale=1.0, outlier=None):
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(H) * scale).astype(np.float32)
    if outlier is not None:
        a[outlier] *= 50
    return bf16_from_f32(a)


def test_int8_hand_example():
    x = bf16_from_f32(np.array([1.0, -0.5, 0.25, 0.0, -1.0, 0.75], np.float32))
    q, s = quant.quant_int8_token(x)
    # m = 127 / 1 = 127; -0.5 * 127 = -63.5 ties to -64 (even); 0.25 * 127 = 31.75 -> 32
    assert q.tolist() == [127, -64, 32, 0, -127, 95]   # 0.75 * 127 = 95.25 -> 95
    assert s == np.float32(1.0) / np.float32(127.0)


@pytest.mark.parametrize("seed", range(5))
def test_int8_properties(seed):
    H = 7168
    x = _row(seed, H, outlier=[3, 100] if seed % 2 else None)
    q, s = quant.quant_int8_token(x)
    xf = codecs.bf16_bits_to_f32(x).astype(np.float64)
    amax = np.max(np.abs(xf))
    assert np.all(np.abs(q.astype(int)) <= 127)
    i = int(np.argmax(np.abs(xf)))
    assert abs(int(q[i])) == 127 and np.sign(q[i]) == np.sign(xf[i])
    assert abs(float(s) - amax / 127) <= 2 ** -23 * amax / 127
    err = np.abs(q.astype(np.float64) * float(s) - xf)
    # half a step plus the float32 roundings of m and x*m
    assert np.all(err <= float(s) * (0.5 + 1e-5) + 1e-6 * np.abs(xf))


def test_int8_zero_and_tiny_rows():
    q, s = quant.quant_int8_token(np.zeros(64, np.uint16))
    assert s == 0 and not q.any()
    tiny = np.full(64, 0x0001, np.uint16)            # smallest bf16 subnormal: 127/amax overflows
    q, s = quant.quant_int8_token(tiny)
    assert s == 0 and not q.any()


def test_fp8_b128_hand_example():
    vals = np.zeros(128, np.float32)
    vals[0], vals[1], vals[2] = 2.0, -1.0, 0.5          # amax 2 -> m = 224
    x = bf16_from_f32(vals)
    codes, scales = quant.quant_fp8_b128(x)
    # 2*224 = 448 -> 0x7E; -224 = -1.75 * 2**7 -> 0xF6; 112 = 1.75 * 2**6 -> 0x6E
    assert codes[0] == 0x7E and codes[1] == 0xF6 and codes[2] == 0x6E and not codes[3:].any()
    assert scales[0] == np.float32(2.0) / np.float32(448.0)


@pytest.mark.parametrize("seed", range(4))
def test_fp8_b128_properties(seed):
    H = 1024
    x = _row(10 + seed, H, scale=10.0 ** (seed - 2))
    codes, scales = quant.quant_fp8_b128(x)
    xf = codecs.bf16_bits_to_f32(x).astype(np.float64)
    v = codecs.e4m3_decode(codes)
    assert np.all(np.abs(v) <= 448)
    for g in range(H // 128):
        blk = xf[g * 128:(g + 1) * 128]
        i = int(np.argmax(np.abs(blk)))
        assert abs(v[g * 128 + i]) == 448.0
        deq = v[g * 128:(g + 1) * 128] * float(scales[g])
        # e4m3 has 3 mantissa bits: relative step 2**-3, half step 2**-4, plus the
        # subnormal floor 2**-10 of the scaled value
        bound = np.maximum(np.abs(blk) * 2 ** -4, 2 ** -10 * float(scales[g])) * (1 + 1e-5)
        assert np.all(np.abs(deq - blk) <= bound + 1e-30)


def _frexp_exponent(amax, emax):
    if amax == 0:
        return -127
    m, e = math.frexp(float(amax))               # amax = m * 2**e, 0.5 <= m < 1
    return max(-127, min(127, (e - 1) - emax))


@pytest.mark.parametrize("mode,emax,vmax", [("mxfp8", 8, 448.0), ("mxfp4", 2, 6.0)])
def test_mx_scale_byte_frexp(mode, emax, vmax):
    rng = np.random.default_rng(3)
    rows = []
    for s in (1e-40, 1e-30, 1e-3, 1.0, 7.0, 1e10, 1e37):   # subnormal to huge
        rows.append((rng.standard_normal(256) * s).astype(np.float32))
    z = np.zeros(256, np.float32)
    z[40:] = rows[3][40:]                        # first block all zero
    rows.append(z)
    for a in rows:
        x = bf16_from_f32(a)
        xf = codecs.bf16_bits_to_f32(x)
        data, sb = quant.quantize_row(mode, x)
        for g in range(256 // 32):
            amax = np.max(np.abs(xf[g * 32:(g + 1) * 32]))
            se = _frexp_exponent(amax, emax)
            assert int(sb[g]) == se + 127
            if amax != 0 and -127 < se < 127:
                scaled = float(amax) * 2.0 ** -se
                assert 2.0 ** emax <= scaled < 2.0 ** (emax + 1)
        codes = data if mode == "mxfp8" else codecs.unpack_e2m1_pairs(data)
        vals = codecs.e4m3_decode(codes) if mode == "mxfp8" else codecs.e2m1_decode(codes)
        assert np.all(np.abs(vals) <= vmax)


def test_mx_zero_block():
    data, sb = quant.quantize_row("mxfp8", np.zeros(64, np.uint16))
    assert sb.tolist() == [0, 0] and not data.any()
    data, sb = quant.quantize_row("mxfp4", np.zeros(64, np.uint16))
    assert sb.tolist() == [0, 0] and not data.any()


@pytest.mark.parametrize("mode,rel", [("int8_token", 0.02), ("fp8_b128", 0.04),
                                      ("mxfp8", 0.05), ("mxfp4", 0.2)])
def test_roundtrip_relative_error(mode, rel):
    H = 7168
    x = _row(20, H)
    d, s = quant.quantize_row(mode, x)
    y = quant.dequantize_row(mode, d, s, H).astype(np.float64)
    xf = codecs.bf16_bits_to_f32(x).astype(np.float64)
    assert np.linalg.norm(y - xf) / np.linalg.norm(xf) < rel


def test_row_bytes():
    assert quant.row_bytes("none", 7168) == (14336, 0)
    assert quant.row_bytes("int8_token", 7168) == (7168, 4)
    assert quant.row_bytes("fp8_b128", 7168) == (7168, 224)
    assert quant.row_bytes("mxfp8", 7168) == (7168, 224)
    assert quant.row_bytes("mxfp4", 7168) == (3584, 224)


# ---------------------------------------------------------------------------
# per-128 e4m3 with power-of-two scales (float32 or e8m0 bytes)
# ---------------------------------------------------------------------------


def _ceil_log2_frexp(v):
    m, e = math.frexp(float(v))                  # v = m * 2**e, 0.5 <= m < 1
    return e - 1 if m == 0.5 else e


def test_ceil_log2_matches_frexp():
    rng = np.random.default_rng(4)
    vals = [np.float32(2.0 ** j) for j in range(-149, 128)]
    vals += [np.nextafter(np.float32(2.0 ** j), np.float32(np.inf)) for j in range(-149, 127)]
    vals += [np.nextafter(np.float32(2.0 ** j), np.float32(0)) for j in range(-148, 128)]
    vals += list(np.abs(rng.standard_normal(2000)).astype(np.float32) * np.float32(1e-30))
    vals += list(np.abs(rng.standard_normal(2000)).astype(np.float32) * np.float32(1e30))
    vals += [np.float32(np.uint32(b).view(np.float32)) for b in (1, 2, 3, 0x7FFFFF, 0x800000, 0x7F7FFFFF)]
    for v in vals:
        assert quant.ceil_log2(v) == _ceil_log2_frexp(v), v


def test_pow2_hand_example():
    vals = np.zeros(256, np.float32)
    vals[:4] = [1.0, -0.5, 0.3, 0.0]               # block 0: amax 1 -> s0 = 1/448 -> scale 2**-8
    vals[128] = 3.0                                 # block 1: s0 = 3/448 -> 2**-7, multiplier 128
    vals[129] = -0.01
    x = bf16_from_f32(vals)
    assert codecs.bf16_bits_to_f32(x)[2] == np.float32(0.30078125)   # bf16(0.3)
    d, s = quant.quantize_row("fp8_b128_pow2", x)
    # 1.0*256 = 256 = 2**8 -> 0x78; -128 -> 0xF0; 0.30078125*256 = 77 -> nearest of 72, 80 is 80 -> 0x6A
    assert d[:4].tolist() == [0x78, 0xF0, 0x6A, 0x00]
    # 3*128 = 384 = 1.5 * 2**8 -> 0x7C; -0.01 (bf16 -0.010009765625) * 128 = -1.28125 -> -1.25 -> 0xBA
    assert d[128] == 0x7C and d[129] == 0xBA
    assert s.view("<f4").tolist() == [2.0 ** -8, 2.0 ** -7]
    d8, b = quant.quantize_row("fp8_b128_ue8m0", x)
    assert np.array_equal(d8, d) and b.tolist() == [127 - 8, 127 - 7]


@pytest.mark.parametrize("seed", range(5))
def test_pow2_scale_properties(seed):
    H = 1024
    x = _row(30 + seed, H, scale=10.0 ** (3 * seed - 6), outlier=[5] if seed % 2 else None)
    xf = codecs.bf16_bits_to_f32(x).astype(np.float64)
    d, s = quant.quantize_row("fp8_b128_pow2", x)
    sc = s.view("<f4").astype(np.float64)
    v = codecs.e4m3_decode(d)
    assert np.all(np.abs(v) <= 448)
    for g in range(H // 128):
        blk = xf[g * 128:(g + 1) * 128]
        amax = np.max(np.abs(blk))
        s0 = float(np.float32(np.float32(amax) / np.float32(448.0)))
        m, _ = math.frexp(sc[g])
        assert m == 0.5                                   # a power of two
        assert sc[g] >= s0 and sc[g] / 2 < s0             # the smallest one >= s0
        i = int(np.argmax(np.abs(blk)))
        assert 224 <= abs(v[g * 128 + i]) <= 448          # the largest element uses the top octave
        deq = v[g * 128:(g + 1) * 128] * sc[g]
        bound = np.maximum(np.abs(blk) * 2 ** -4, 2 ** -10 * sc[g]) * (1 + 1e-6)
        assert np.all(np.abs(deq - blk) <= bound + 1e-300)
    d8, b = quant.quantize_row("fp8_b128_ue8m0", x)
    assert np.array_equal(d8, d)
    assert np.array_equal(codecs.e8m0_decode(b), sc)


def test_pow2_reduces_to_fp8_b128_when_scale_is_a_power_of_two():
    rng = np.random.default_rng(8)
    H = 512
    a = rng.uniform(-1, 1, H).astype(np.float32)
    for g, j in enumerate([0, -3, 5, -20]):
        a[g * 128:(g + 1) * 128] *= np.float32(2.0 ** j)  # |elements| < 2**j
        a[g * 128 + 7] = np.float32(448.0 * 2.0 ** j)     # amax 448 * 2**j: s0 = 2**j exactly
    x = bf16_from_f32(a)
    d0, s0 = quant.quantize_row("fp8_b128", x)
    d1, s1 = quant.quantize_row("fp8_b128_pow2", x)
    assert np.array_equal(d0, d1) and np.array_equal(s0, s1)


def test_pow2_zero_tiny_and_boundary_blocks():
    z = np.zeros(128, np.uint16)
    for mode, sb in [("fp8_b128_pow2", 4), ("fp8_b128_ue8m0", 1)]:
        d, s = quant.quantize_row(mode, z)
        assert not d.any() and not s.any() and s.size == sb
        d, s = quant.quantize_row(mode, np.full(128, 0x0001, np.uint16))   # amax 2**-133: e < -127
        assert not d.any() and not s.any()
    # amax = 448 * 2**-127: e = -127 exactly, the last block that is kept
    edge = np.zeros(128, np.float32)
    edge[0] = np.float32(1.75 * 2.0 ** -119)
    d, b = quant.quantize_row("fp8_b128_ue8m0", bf16_from_f32(edge))
    assert d[0] == 0x7E and b[0] == 0
    d, s = quant.quantize_row("fp8_b128_pow2", bf16_from_f32(edge))
    assert d[0] == 0x7E and s.view("<f4")[0] == np.float32(2.0 ** -127)
    # half of that: e = -128, the multiplier 2**128 overflows -> zero block
    edge[0] = np.float32(1.75 * 2.0 ** -120)
    d, b = quant.quantize_row("fp8_b128_ue8m0", bf16_from_f32(edge))
    assert not d.any() and b[0] == 0


@pytest.mark.parametrize("mode", ["fp8_b128_pow2", "fp8_b128_ue8m0"])
def test_pow2_roundtrip_relative_error(mode):
    H = 7168
    x = _row(21, H)
    d, s = quant.quantize_row(mode, x)
    y = quant.dequantize_row(mode, d, s, H).astype(np.float64)
    xf = codecs.bf16_bits_to_f32(x).astype(np.float64)
    assert np.linalg.norm(y - xf) / np.linalg.norm(xf) < 0.05
    assert quant.row_bytes(mode, H) == (H, 224 if mode.endswith("pow2") else 56)
