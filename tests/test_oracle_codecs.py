"""Pins of the oracle's element codecs against things other than itself.

* bf16 rounding and e4m3fn rounding: torch's CPU casts (library routines),
  over every bfloat16 pattern, every midpoint and random float32 values.
* e2m1: a midpoint table written out by hand from the OCP value list
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}, and brute-force nearest search over all 16
  codes.
* decoders: exhaustive closed forms.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _all_bf16_f32(finite=True):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_bits_to_f32(b)
    return f[np.isfinite(f)] if finite else f


def test_bf16_widen_is_exact_on_every_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_bits_to_f32(b)
    back = f.view(np.uint32)
    assert np.array_equal(back >> 16, b.astype(np.uint32))
    assert np.all((back & 0xFFFF) == 0)


def test_bf16_round_matches_torch_on_values_midpoints_and_random():
    vals = _all_bf16_f32()
    # midpoints between consecutive positive bf16 patterns (exact ties)
    pos = np.arange(0, 0x7F7F, dtype=np.uint32)
    mid = ((pos << 16) + 0x8000).view(np.float32)
    rng = np.random.default_rng(0)
    rand = rng.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    big = np.array([3.3895314e38, 3.39e38, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 0.0, -0.0],
                   np.float32)
    for x in (vals, mid, -mid, rand, bits, big):
        assert np.array_equal(codecs.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_round_nan_is_quiet_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    r = codecs.f32_to_bf16_bits(x)
    assert np.all((r & 0x7FFF) == 0x7FC0)


def test_bf16_round_ties_to_even_examples():
    # 1 + 2**-8 lies halfway between 1 and 1 + 2**-7; the even neighbour is 1.
    assert codecs.f32_to_bf16_bits(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3 * 2**-8 lies halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even).
    assert codecs.f32_to_bf16_bits(np.float32(1 + 3 * 2 ** -8)) == 0x3F82


def test_e4m3_decode_closed_form():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    v = codecs.e4m3_decode(codes)
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(v[nan])) and not np.any(np.isnan(v[~nan]))
    # the same values as torch's widening of float8_e4m3fn
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(v[~nan].astype(np.float32), ref[~nan])
    # a few hand-checked points: smallest subnormal, smallest normal, 1, max
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    assert v[0xFE] == -448.0 and v[0x80] == 0.0 and np.signbit(v[0x80])


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(1)
    vals = _all_bf16_f32()
    vals = vals[np.abs(vals) <= 448.0]
    pos = codecs.E4M3_POS_VALUES
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)        # exact in float32
    just = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rand = (rng.random(300000) * 896 - 448).astype(np.float32)
    tiny = (rng.standard_normal(100000) * 2 ** -8).astype(np.float32)
    special = np.array([0.0, -0.0, -1e-6, 1e-6, 448.0, -448.0, 2 ** -10, -(2 ** -10)], np.float32)
    for x in (vals, mids, -mids, just, -just, rand, tiny, special):
        x = np.clip(x, np.float32(-448), np.float32(448))
        assert np.array_equal(codecs.e4m3_encode(x), _torch_e4m3_bits(x))


def test_e4m3_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([449.0], np.float32))


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    v = codecs.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(codecs.e4m3_encode(v), codes)


E2M1_TABLE = [
    # value, expected code (hand-written from the OCP list 0, .5, 1, 1.5, 2, 3, 4, 6)
    (0.0, 0x0), (0.25, 0x0), (0.2500001, 0x1), (0.5, 0x1), (0.75, 0x2), (0.74999994, 0x1),
    (1.0, 0x2), (1.25, 0x2), (1.2500001, 0x3), (1.5, 0x3), (1.75, 0x4), (2.0, 0x4),
    (2.5, 0x4), (2.5000002, 0x5), (3.0, 0x5), (3.5, 0x6), (3.4999998, 0x5), (4.0, 0x6),
    (5.0, 0x6), (5.0000005, 0x7), (6.0, 0x7), (-0.0, 0x8), (-0.1, 0x8), (-0.75, 0xA),
    (-5.0, 0xE), (-6.0, 0xF),
]


def test_e2m1_encode_hand_table():
    x = np.array([v for v, _ in E2M1_TABLE], np.float32)
    want = np.array([c for _, c in E2M1_TABLE], np.uint8)
    assert np.array_equal(codecs.e2m1_encode(x), want)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(2)
    x = (rng.random(20000) * 12 - 6).astype(np.float32)
    got = codecs.e2m1_encode(x)
    allc = np.arange(16, dtype=np.uint8)
    allv = codecs.e2m1_decode(allc)
    for xi, ci in zip(x[:4000], got[:4000]):
        d = np.abs(allv - float(xi))
        best = d.min()
        cands = [int(c) for c in allc if d[c] == best and (np.signbit(allv[c]) == np.signbit(xi) or allv[c] != 0)]
        assert int(ci) in cands
        if len(cands) > 1:            # a tie: the chosen code is the even one
            assert int(ci) % 2 == 0


def test_e2m1_pack_order_low_nibble_first():
    codes = np.array([0x1, 0x7, 0xA, 0x3], np.uint8)
    p = codecs.pack_e2m1_pairs(codes)
    assert list(p) == [0x71, 0x3A]
    assert np.array_equal(codecs.unpack_e2m1_pairs(p), codes)


def test_e8m0_decode():
    b = np.array([0, 1, 126, 127, 128, 254, 255], np.uint8)
    v = codecs.e8m0_decode(b)
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 0.5 and v[3] == 1.0
    assert v[4] == 2.0 and v[5] == 2.0 ** 127 and np.isnan(v[6])
