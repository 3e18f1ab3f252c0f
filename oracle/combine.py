"""Combine of the oracle (test infrastructure only).

For each token t ("Low-Latency Mode API", ``low_latency_combine``: the result
is the bf16 weighted sum of the token's expert outputs; "DeepEP FP8 Dispatch
and Combine Operations", "The FP8 Combine Operation": codes are multiplied
by the stored inverse scale through float32 and accumulated):

    acc = +0.0 (float32)
    for j = 0 .. k-1, skipping pairs with slot[t, j] == -1:
        y   = dequantised row slot[t, j]      (float32, ``quant.dequantize_row``)
        p   = fl32(topk_weights[t, j] * y)
        acc = fl32(acc + p)
    out[t] = bf16 round-half-even of acc

One multiply then one add per term, float32, no fused multiply-add and no
reordering (one page describes the accumulation as bf16 in one place and as
going through float32 in another; float32 accumulation, rounded once, is the
reading taken).  A token with no
routed pair gives +0 (the pages are silent on this case).

Parity: pinned by the closed form for unit weights and bf16 rows (the sum
of k_eff equal terms is exact in float32, so out == bf16(k_eff * x)), and for
general weights by the bound "within one bf16 ulp of the float64 sum"
(see ``tests/test_oracle_path.py``).
"""

from __future__ import annotations

import numpy as np

from . import codecs, quant
from .dispatch import RecvBuffer
from .layout import Layout


def combine_token(expert_out: RecvBuffer, lay: Layout, topk_weights: np.ndarray, t: int) -> np.ndarray:
    """float32 accumulator of token t (before the bf16 rounding)."""
    H = expert_out.hidden
    acc = np.zeros(H, np.float32)
    for j in range(lay.num_topk):
        r = int(lay.slot[t, j])
        if r < 0:
            continue
        y = quant.dequantize_row(expert_out.mode, expert_out.data[r], expert_out.scales[r], H)
        w = np.float32(topk_weights[t, j])
        with np.errstate(over="ignore", invalid="ignore"):
            p = (w * y).astype(np.float32)
            acc = (acc + p).astype(np.float32)
    return acc


def combine(expert_out: RecvBuffer, lay: Layout, topk_weights: np.ndarray, tokens=None) -> np.ndarray:
    """bf16 patterns (uint16) [T, H], or [len(tokens), H] for a sample."""
    topk_weights = np.asarray(topk_weights, dtype=np.float32)
    ts = range(lay.num_tokens) if tokens is None else [int(t) for t in tokens]
    out = np.zeros((len(ts), expert_out.hidden), np.uint16)
    for i, t in enumerate(ts):
        out[i] = codecs.f32_to_bf16_bits(combine_token(expert_out, lay, topk_weights, t))
    return out
