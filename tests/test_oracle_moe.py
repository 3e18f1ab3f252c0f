"""Pins of the oracle's expert MLP (GMM1 -> SwiGLU -> requant -> GMM2).

* MX dequantisation: scale byte 127 reproduces the (pinned) e4m3 decode, and
  byte 127 + j multiplies it by exactly 2**j;
* dot products: ``numpy.matmul`` against brute-force Python loops on small
  inputs;
* silu: against ``z * scipy.special.expit(z)`` and its limits;
* gate/up split and both transposes: one-hot weights turn the MLP into the
  closed form a_n = silu(x[p(n)]) * x[q(n)], y_m = deq(q)[s(m)]; swapping the
  two halves of W1 or transposing an operand gives a different result (the
  planted mistakes below are caught);
* requant: on float32 inputs that are bf16 values it equals the pinned bf16
  MXFP8 quantiser.
"""

import math

import numpy as np
import pytest
from scipy.special import expit

from combine_topk_idx_amd.workloads import bf16_from_f32, make_mx_weights
from oracle import codecs, moe, quant

ONE = 0x38            # e4m3 code of 1.0


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x30        # no NaN codes
    return c


def test_mx_dequant_scale_bytes():
    rng = np.random.default_rng(1)
    codes = _rand_codes(rng, (3, 64))
    base = codecs.e4m3_decode(codes)
    assert np.array_equal(moe.mx_dequant(codes, np.full((3, 2), 127, np.uint8)), base)
    for j in (-20, -3, 1, 9):
        s = np.full((3, 2), 127 + j, np.uint8)
        assert np.array_equal(moe.mx_dequant(codes, s), base * 2.0 ** j)
    s = np.array([[127, 130]] * 3, np.uint8)                 # each byte covers its own 32 codes
    d = moe.mx_dequant(codes, s)
    assert np.array_equal(d[:, :32], base[:, :32]) and np.array_equal(d[:, 32:], base[:, 32:] * 8)


def test_silu_against_expit():
    z = np.concatenate([np.linspace(-40, 40, 2001), [0.0, 1e-8, -1e-8, 700.0, -700.0, -1000.0]])
    assert np.allclose(moe.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert moe.silu(np.array([0.0]))[0] == 0.0
    assert moe.silu(np.array([-1000.0]))[0] == 0.0            # the limit, no NaN
    assert moe.silu(np.array([50.0]))[0] == pytest.approx(50.0, rel=1e-15)


def _brute_dot_rows(xv, wv):
    R, K = xv.shape
    N = wv.shape[0]
    out = np.zeros((R, N))
    for r in range(R):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(xv[r, k]) * float(wv[n, k])
            out[r, n] = s
    return out


def test_gmm1_and_gmm2_against_brute_force():
    rng = np.random.default_rng(2)
    R, H, I = 3, 64, 32
    xc, xs = _rand_codes(rng, (R, H)), rng.integers(120, 130, (R, H // 32)).astype(np.uint8)
    w1c, w1s = _rand_codes(rng, (2 * I, H)), rng.integers(118, 125, (2 * I, H // 32)).astype(np.uint8)
    w2c, w2s = _rand_codes(rng, (H, I)), rng.integers(118, 125, (H, I // 32)).astype(np.uint8)
    _, _, a = moe.gmm1_swiglu_rows(xc, xs, w1c, w1s, "bf16")
    xv, w1v = moe.mx_dequant(xc, xs), moe.mx_dequant(w1c, w1s)
    gu = _brute_dot_rows(xv, w1v)
    g, u = gu[:, :I], gu[:, I:]
    want = np.array([[gg * float(expit(gg)) * uu for gg, uu in zip(gr, ur)] for gr, ur in zip(g, u)])
    assert np.allclose(a, want, rtol=1e-12, atol=1e-300)
    q, qs, _ = moe.gmm1_swiglu_rows(xc, xs, w1c, w1s, "mxfp8")
    bits, y = moe.gmm2_rows(q, qs, w2c, w2s)
    yb = _brute_dot_rows(moe.mx_dequant(q, qs), moe.mx_dequant(w2c, w2s))
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-300)
    assert np.array_equal(bits, codecs.f32_to_bf16_bits(yb.astype(np.float32)))


def _one_hot(rows, K, cols):
    c = np.zeros((rows, K), np.uint8)
    c[np.arange(rows), cols] = ONE
    return c, np.full((rows, K // 32), 127, np.uint8)


def test_one_hot_closed_form_and_planted_mistakes():
    rng = np.random.default_rng(3)
    R, H, I = 5, 64, 32
    x = bf16_from_f32(rng.standard_normal((R, H)).astype(np.float32))
    xc, xs = np.empty((R, H), np.uint8), np.empty((R, H // 32), np.uint8)
    for r in range(R):
        xc[r], xs[r] = quant.quant_mxfp8(x[r])
    xv = moe.mx_dequant(xc, xs)
    p = rng.permutation(H)[:I]               # gate row n reads x[p[n]]
    q = rng.permutation(H)[:I]               # up row n reads x[q[n]]
    w1c, w1s = _one_hot(2 * I, H, np.concatenate([p, q]))
    _, _, a = moe.gmm1_swiglu_rows(xc, xs, w1c, w1s, "bf16")
    want = moe.silu(xv[:, p]) * xv[:, q]
    assert np.array_equal(a, want)
    # planted: gate and up swapped, or W1 read transposed, gives something else
    swapped = moe.silu(xv[:, q]) * xv[:, p]
    assert not np.allclose(a, swapped)
    qc, qsc, _ = moe.gmm1_swiglu_rows(xc, xs, w1c, w1s, "mxfp8")
    s = rng.permutation(I)
    w2c, w2s = _one_hot(H, I, np.resize(s, H))
    bits, y = moe.gmm2_rows(qc, qsc, w2c, w2s)
    assert np.array_equal(y, moe.mx_dequant(qc, qsc)[:, np.resize(s, H)])


def test_requant_equals_bf16_quantiser_on_bf16_values():
    rng = np.random.default_rng(4)
    for scale in (1e-30, 1e-3, 1.0, 1e6):
        xb = bf16_from_f32((rng.standard_normal(256) * scale).astype(np.float32))
        xf = codecs.bf16_bits_to_f32(xb)
        a = quant.quant_mxfp8_f32(xf)
        b = quant.quant_mxfp8(xb)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_synthetic_weights_are_finite_mx():
    c, s = make_mx_weights(5, 2, 64, 256)
    assert c.shape == (2, 64, 256) and s.shape == (2, 64, 8)
    assert not np.any((c & 0x7F) == 0x7F)
    v = moe.mx_dequant(c, s)
    assert np.all(np.isfinite(v)) and 0.1 < np.std(v) * math.sqrt(256) < 10
