"""GPU: the precision model of the MX-scaled matrix-core step that the
expert-MLP bounds rest on (``tests/moe_bounds.py``).

Model: one v_mfma_scale_f32_32x32x64_f8f6f4 step (e4m3 x e4m3, an e8m0 scale
per 32-element block of each operand) returns c0 + sum_k a_k b_k with an
error of at most 2^-11 of the step's largest |a_k b_k| (at least 11 fraction
bits below the leading bit of its largest product), then rounded to float32.

Each case runs one step through ``ep_probe_mfma`` (libep_probe.so) and is
compared with the exact sum (Python integers): 4000 seeded random blocks
(every finite e4m3 code, block scales 2^-9 .. 2^9, with and without an
accumulator input), blocks whose largest product dwarfs the rest (the
smallest terms then fall out of the step's window) and cross-block sums
whose terms cancel.  The largest error seen, as a fraction of the model's
allowance, is printed.
"""

import ctypes
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import build as B

pytestmark = pytest.mark.gpu

REC = np.dtype([("a", np.uint8, 64), ("b", np.uint8, 64), ("sa", np.uint8, 2), ("sb", np.uint8, 2),
                ("c0", "<f4")])
FRAC_BITS = 11
ONE, MINUS_ONE, MAX, MINUS_MAX = 0x38, 0xB8, 0x7E, 0xFE


def _value(code: int) -> Fraction:
    """e4m3 code -> exact value (OCP e4m3fn: bias 7, no infinity)."""
    s = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return s * Fraction(m, 8) / 64
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


VALUES = [_value(c) for c in range(256)]


def _cases(seed=11, n_random=4000):
    rng = np.random.default_rng(seed)
    out = []
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    for i in range(n_random):
        r = np.zeros((), REC)
        r["a"], r["b"] = rng.choice(finite, 64), rng.choice(finite, 64)
        r["sa"], r["sb"] = rng.integers(118, 137, 2), rng.integers(118, 137, 2)
        r["c0"] = 0.0 if i % 2 == 0 else np.float32(rng.standard_normal() * 64)
        out.append(r)
    for code in range(1, 0x7F):                       # 448*448 and a smaller term in one block
        for a in ({0: MAX, 1: MINUS_MAX, 2: code}, {0: MAX, 2: code}, {0: MAX, 2: code | 0x80}):
            r = np.zeros((), REC)
            r["b"] = ONE
            for k, v in a.items():
                r["a"][k] = v
            r["sa"], r["sb"] = (127, 127), (127, 127)
            out.append(r)
    for m in range(0, 60):                            # cross-block: +-1 in block 0, 2^-m in block 1
        for a in ({0: ONE, 1: MINUS_ONE, 32: ONE}, {0: ONE, 32: ONE}, {0: ONE, 32: MINUS_ONE}):
            r = np.zeros((), REC)
            r["b"] = ONE
            for k, v in a.items():
                r["a"][k] = v
            r["sa"], r["sb"] = (127, max(127 - m, 0)), (127, 127)
            out.append(r)
    return np.array(out, dtype=REC)


def _exact(rec):
    """(exact result, largest |product|) of one case."""
    tot = Fraction(float(rec["c0"]))
    big = Fraction(0)
    for k in range(64):
        blk = k // 32
        p = VALUES[int(rec["a"][k])] * VALUES[int(rec["b"][k])] * \
            Fraction(2) ** (int(rec["sa"][blk]) + int(rec["sb"][blk]) - 254)
        tot += p
        big = max(big, abs(p))
    return tot, big


def test_step_error_within_the_model():
    print("\n[case] MFMA step precision model", flush=True)
    sys.stdout.flush()
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.ep_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    cases = _cases()
    n = cases.size
    d_cases = torch.from_numpy(cases.view(np.uint8).copy()).cuda()
    d_out = torch.empty(n * 64, dtype=torch.float32, device="cuda")
    assert lib.ep_probe_mfma(d_cases.data_ptr(), n, d_out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    got = d_out.view(n, 64)[:, 0].cpu().numpy()
    worst, worst_i, inexact = 0.0, -1, 0
    for i in range(n):
        ex, big = _exact(cases[i])
        allow = Fraction(2) ** -FRAC_BITS * big
        # the float32 rounding of the accumulator, on top of the model
        r32 = (abs(ex) + allow) * Fraction(2) ** -24 + Fraction(2) ** -149
        err = abs(Fraction(float(got[i])) - ex)
        inexact += err > r32
        assert err <= allow + r32, (f"case {i}: got {got[i]!r}, exact {float(ex)!r}, error {float(err):.3g} > "
                                    f"2^-{FRAC_BITS} x largest product {float(big):.3g}")
        if allow > 0 and err > r32:
            ratio = float((err - r32) / allow)
            if ratio > worst:
                worst, worst_i = ratio, i
    print(f"{n} steps, {inexact} off the float32-rounded exact sum; worst error {worst:.3f} of the model's "
          f"allowance (case {worst_i})")
    # the model is not vacuous: the device does lose precision inside a step
    assert inexact > 0
