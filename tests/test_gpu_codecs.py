"""GPU: the element converters of the library (``csrc/formats.hpp`` and the
scaled bf16 -> e4m3 conversion of the weighted reverse dispatch) against the
oracle's software codecs, bit for bit, over their whole input domains.

They run through ``ep_probe_codec`` of libep_probe.so, which calls the same
inline functions the kernels call:

* e4m3 and e2m1 decoding times a power-of-two scale: every code with every
  e8m0 scale byte (products past float32's range are +-inf, byte 0xFF NaN);
* e2m1 encoding of bf16 divided by a power of two, and the scaled e4m3
  encoding of bf16 (inputs clamped to +-448 times the scale, as the kernel
  does): every finite bf16 pattern with every scale exponent -127 .. 126;
* e4m3 encoding of float32 within +-448: every bf16 value, every rounding
  midpoint and its float32 neighbours, and 2^22 random float32;
* bf16 packing of float32: every bf16 pattern with the low halves 0, 1,
  0x7FFF, 0x8000, 0x8001 and 0xFFFF (every tie and its neighbours), and
  +-inf.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import build as B
from oracle import codecs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.ep_probe_codec.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_void_p]
    return lib


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _run(lib, kind, inp: np.ndarray, groups: int, out_dtype, out_count: int, scale: float = 1.0) -> np.ndarray:
    d_in = torch.from_numpy(np.ascontiguousarray(inp).view(np.uint8).copy()).cuda()
    d_out = torch.zeros(out_count * np.dtype(out_dtype).itemsize, dtype=torch.uint8, device="cuda")
    rc = lib.ep_probe_codec(kind, d_in.data_ptr(), d_out.data_ptr(), groups, scale,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return d_out.cpu().numpy().view(out_dtype)


def _pow2_f32(e: int) -> np.float32:
    """2^e as float32, e in [-127, 127] (2^-127 is the subnormal 0x00400000)."""
    bits = 0x00400000 if e == -127 else (e + 127) << 23
    return np.array([bits], np.uint32).view(np.float32)[0]


def _finite_bf16() -> np.ndarray:
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return pats[np.isfinite(codecs.bf16_bits_to_f32(pats))]


def _same_float_bits(got: np.ndarray, want: np.ndarray):
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn)
    assert np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


def test_e4m3_decode_every_code_and_scale(lib):
    _announce("e4m3 decode x e8m0, every pair")
    code = np.arange(65536, dtype=np.uint32) & 0xFF
    byte = np.arange(65536, dtype=np.uint32) >> 8
    got = _run(lib, 1, (code | (byte << 8)).astype(np.uint16), 65536, np.float32, 65536)
    with np.errstate(over="ignore", invalid="ignore"):
        want = (codecs.e4m3_decode(code.astype(np.uint8)) * codecs.e8m0_decode(byte.astype(np.uint8))).astype(np.float32)
    _same_float_bits(got, want)


def test_e2m1_decode_every_code_and_scale(lib):
    _announce("e2m1 decode x e8m0, every pair")
    code = np.tile(np.arange(16, dtype=np.uint32), 256)
    byte = np.repeat(np.arange(256, dtype=np.uint32), 16)
    got = _run(lib, 3, (code | (byte << 8)).astype(np.uint16), code.size, np.float32, code.size)
    with np.errstate(over="ignore", invalid="ignore"):
        want = (codecs.e2m1_decode(code.astype(np.uint8)) * codecs.e8m0_decode(byte.astype(np.uint8))).astype(np.float32)
    _same_float_bits(got, want)


def _pad8(a: np.ndarray) -> np.ndarray:
    return np.concatenate([a, np.zeros((-a.size) % 8, a.dtype)])


def test_e2m1_encode_every_bf16_and_scale(lib):
    _announce("e2m1 encode of bf16 / 2^e, every finite bf16 and e")
    x = _pad8(_finite_bf16())
    xv = codecs.bf16_bits_to_f32(x).astype(np.float64)
    for e in range(-127, 127):
        got = _run(lib, 2, x, x.size // 8, np.uint32, x.size // 8, _pow2_f32(e))
        nib = ((got[:, None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF).astype(np.uint8).reshape(-1)
        want = codecs.e2m1_encode(np.clip(xv / 2.0 ** e, -6.0, 6.0).astype(np.float32))
        bad = nib != want
        assert not bad.any(), (f"e = {e}: {bad.sum()} codes differ; first bf16 {x[bad][0]:#06x}: "
                               f"got {nib[bad][0]:#x}, want {want[bad][0]:#x}")


def test_scaled_e4m3_from_bf16_every_input_and_scale(lib):
    """The reverse dispatch's conversion: bf16 inputs already clamped to
    +-448 * 2^e, divided by 2^e and rounded to e4m3."""
    _announce("scaled e4m3 of bf16 / 2^e, every finite bf16 and e")
    x0 = _finite_bf16()
    v0 = codecs.bf16_bits_to_f32(x0).astype(np.float64)
    for e in range(-127, 127):
        lim = 448.0 * 2.0 ** e
        v = np.clip(v0, -lim, lim) if lim < 2.0 ** 128 else v0      # past float32's range: no clamp
        x = _pad8(codecs.f32_to_bf16_bits(v.astype(np.float32)))   # the clamp limit is a bf16 value
        vx = codecs.bf16_bits_to_f32(x).astype(np.float64)
        got = _run(lib, 5, x, x.size // 8, np.uint8, x.size, _pow2_f32(e))
        want = codecs.e4m3_encode(np.clip(vx / 2.0 ** e, -448.0, 448.0).astype(np.float32))
        bad = got != want
        assert not bad.any(), (f"e = {e}: {bad.sum()} codes differ; first bf16 {x[bad][0]:#06x}: "
                               f"got {got[bad][0]:#x}, want {want[bad][0]:#x}")


def test_scaled_e4m3_with_a_scalar_scale_operand(lib):
    """The same conversion with the scale read from a scalar register (the
    form a compiler may pick for a workgroup-uniform scale): identical to the
    vector-register form for every input and exponent, the subnormal scale
    2^-127 included."""
    _announce("scaled e4m3 of bf16 / 2^e, scale in a scalar register")
    x = _pad8(_finite_bf16())
    differ = []
    for e in range(-127, 127):
        vec = _run(lib, 5, x, x.size // 8, np.uint8, x.size, _pow2_f32(e))
        sca = _run(lib, 6, x, x.size // 8, np.uint8, x.size, _pow2_f32(e))
        if not np.array_equal(vec, sca):
            differ.append(e)
    assert not differ, f"exponents where the scalar-register form differs: {differ}"


def test_e4m3_encode_float32(lib):
    _announce("e4m3 encode of float32 within +-448")
    rng = np.random.default_rng(5)
    mags = codecs.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)           # exact in float32
    ties = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    rand = (np.exp2(rng.uniform(-14, np.log2(448.0), 1 << 22)) * rng.choice([-1.0, 1.0], 1 << 22)).astype(np.float32)
    allbf = codecs.bf16_bits_to_f32(_finite_bf16())
    v = np.concatenate([ties, -ties, rand, np.clip(allbf, -448, 448)]).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    v = _pad8(v)
    got = _run(lib, 0, v, v.size // 8, np.uint8, v.size)
    want = codecs.e4m3_encode(v)
    bad = got != want
    assert not bad.any(), f"{bad.sum()} codes differ; first {v[bad][0]!r}: got {got[bad][0]:#x}, want {want[bad][0]:#x}"


def test_bf16_pack(lib):
    _announce("bf16 packing of float32")
    hi = np.arange(65536, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]                                # no Inf/NaN halves
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).reshape(-1)
    f = np.concatenate([bits.view(np.float32), np.float32([np.inf, -np.inf])])
    f = np.concatenate([f, np.zeros(f.size % 2, np.float32)])
    got = _run(lib, 4, f, f.size // 2, np.uint32, f.size // 2)
    g = np.stack([got & 0xFFFF, got >> 16], axis=1).reshape(-1).astype(np.uint16)
    want = codecs.f32_to_bf16_bits(f)
    bad = g != want
    assert not bad.any(), f"{bad.sum()} differ; first {f[bad][0]!r}: got {g[bad][0]:#06x}, want {want[bad][0]:#06x}"
