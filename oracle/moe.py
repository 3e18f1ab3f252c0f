"""Expert MLP of the fused MoE operator (test infrastructure only).

"[feat] A5 deep fused moe" describes one operator that runs dispatch, the
first grouped matrix multiply (GMM1), SwiGLU, a requantisation, the second
grouped matrix multiply (GMM2) and combine (Testing: the per-stage timing
table; Benchmarking and Profiling: hidden 7168, moe-intermediate-size 3072,
top-6, FP8 quantisation, uniform routing); its review adds that the GMM1 A
operand is e4m3 with one e8m0 scale per 32-element group.  For expert e and
each receive row r of its block, the oracle computes (readings where the page
is silent are marked *):

    x    = the dequantised MXFP8 dispatch row                      (exact)
    g_n  = sum_h W1[e, n, h] * x_h,      n in [0, I)     gate      (* first half of W1)
    u_n  = sum_h W1[e, I + n, h] * x_h,  n in [0, I)     up
    a_n  = silu(g_n) * u_n,   silu(z) = z / (1 + exp(-z))          (* SwiGLU)
    q    = MXFP8 of fl32(a), per 32 along I, the OCP MX rule of dispatch (Requant)
    y_m  = sum_i W2[e, m, i] * deq(q)_i,  m in [0, H)               (GMM2)
    out  = bf16_rne(fl32(y))                                       (* expert rows in bf16)

W1 [E, 2I, H] and W2 [E, H, I] are MXFP8 like the A operand (* the page fixes
only the A operand's format): e4m3 codes with one e8m0 scale per 32
consecutive elements of the reduction axis.  Every dot product is formed in
float64 from the exact dequantised values and silu in float64; a and y are
rounded to float32 (the precision the GPU accumulates in), a is then
requantised and y rounded to bf16.  The bf16 variant of GMM1
(``out_mode="bf16"``) rounds fl32(a) to bf16 instead of requantising it.

Parity: the dot products are ``numpy.matmul`` over exact float64 values,
pinned against brute-force loops on small inputs; silu against
``z * scipy.special.expit(z)``; the gate/up split and both transposes by
one-hot weights that turn the MLP into a closed form; the requant inherits
the MX rule's pins (``quant``) and is pinned to it by equality on inputs that
are bf16 values; see ``tests/test_oracle_moe.py``.
"""

from __future__ import annotations

import numpy as np

from . import codecs, quant


def mx_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values of MXFP8 data: codes [..., K] e4m3, scales [..., K/32]
    e8m0 bytes (each scale covers 32 consecutive codes).  Exact."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    if codes.shape[-1] != 32 * scales.shape[-1]:
        raise ValueError("one scale byte per 32 codes")
    v = codecs.e4m3_decode(codes)
    s = np.repeat(codecs.e8m0_decode(scales), 32, axis=-1)
    return v * s


def silu(z: np.ndarray) -> np.ndarray:
    """z / (1 + exp(-z)) in float64 (exp overflow for very negative z gives
    the limit 0)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gmm1_swiglu_rows(x_codes: np.ndarray, x_scales: np.ndarray, w1_codes: np.ndarray, w1_scales: np.ndarray,
                     out_mode: str = "mxfp8"):
    """GMM1 + SwiGLU (+ requant) of the rows of one expert.

    x_codes [R, H], x_scales [R, H/32]; w1_codes [2I, H], w1_scales [2I, H/32].
    Returns (data, scales): out_mode "mxfp8" -> e4m3 codes [R, I] and e8m0
    bytes [R, I/32]; "bf16" -> bf16 patterns (uint16) [R, I] and an empty
    scale array.  Also returns the float64 pre-rounding activations a [R, I].
    """
    x = mx_dequant(x_codes, x_scales)
    w = mx_dequant(w1_codes, w1_scales)
    inter = w.shape[0] // 2
    g = x @ w[:inter].T
    u = x @ w[inter:].T
    a = silu(g) * u
    a32 = a.astype(np.float32)
    R = a.shape[0]
    if out_mode == "bf16":
        return codecs.f32_to_bf16_bits(a32), np.zeros((R, 0), np.uint8), a
    if out_mode != "mxfp8":
        raise ValueError(out_mode)
    data = np.empty((R, inter), np.uint8)
    sc = np.empty((R, inter // 32), np.uint8)
    for r in range(R):
        data[r], sc[r] = quant.quant_mxfp8_f32(a32[r])
    return data, sc, a


def gmm2_rows(a_codes: np.ndarray, a_scales: np.ndarray, w2_codes: np.ndarray, w2_scales: np.ndarray):
    """GMM2 of the rows of one expert: a [R, I] MXFP8, w2 [H, I] MXFP8 ->
    (bf16 patterns [R, H], float64 y [R, H])."""
    a = mx_dequant(a_codes, a_scales)
    w = mx_dequant(w2_codes, w2_scales)
    y = a @ w.T
    return codecs.f32_to_bf16_bits(y.astype(np.float32)), y


def abs_products(x_codes, x_scales, w_codes, w_scales) -> np.ndarray:
    """sum_k |x_k * w_k| for every (row, weight row): the scale of the
    rounding error of a dot product, used by the parity bounds."""
    return np.abs(mx_dequant(x_codes, x_scales)) @ np.abs(mx_dequant(w_codes, w_scales)).T
