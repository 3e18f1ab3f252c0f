"""Backward of combine with respect to the expert outputs, as a reverse
dispatch (test infrastructure only; see package header).

"EP dispatch with unfused MXFP8 quantization" (Description and Changes): the
result gradient of combine is scattered back to the expert positions through
the same dispatch operation, quantised.  The combine here computes
out[t] = sum_j w[t, j] * y[slot[t, j]], so the gradient of out[t] with
respect to row slot[t, j] is w[t, j] * grad[t].  With weights the oracle
forms that product in float32 (one rounding), rounds it to bf16 (the expert
output type) and quantises the row like dispatch does; without weights the
rows are dispatch's rows of grad itself.

Parity: pinned by (a) unit weights giving exactly the unweighted rows, (b)
bf16 rows equal to torch's float32 product rounded by torch's bf16 cast,
and (c) the adjoint identity sum_t <grad[t], combine(y)[t]> =
sum_r <dy[r], y[r]> on bf16 rows, within the bf16 rounding of dy (see
``tests/test_oracle_backward.py``).
"""

from __future__ import annotations

import numpy as np

from . import codecs, quant
from .dispatch import RecvBuffer
from .layout import Layout


def scaled_grad_row(grad_bits: np.ndarray, w: float) -> np.ndarray:
    """bf16 patterns of bf16_rne(fl32(w * grad))."""
    g = codecs.bf16_bits_to_f32(grad_bits)
    return codecs.f32_to_bf16_bits((np.float32(w) * g).astype(np.float32))


def combine_backward(grad_bits: np.ndarray, lay: Layout, mode: str,
                     topk_weights: np.ndarray | None = None, tokens=None) -> RecvBuffer:
    grad_bits = np.asarray(grad_bits, dtype=np.uint16)
    T, H = grad_bits.shape
    dq, sq = quant.row_bytes(mode, H)
    data = np.zeros((lay.max_rows, dq), np.uint8)
    scales = np.zeros((lay.max_rows, sq), np.uint8)
    ts = range(T) if tokens is None else [int(t) for t in tokens]
    for t in ts:
        routed = [j for j in range(lay.num_topk) if lay.slot[t, j] >= 0]
        if not routed:
            continue
        if topk_weights is None:
            d, s = quant.quantize_row(mode, grad_bits[t])
        for j in routed:
            if topk_weights is not None:
                d, s = quant.quantize_row(mode, scaled_grad_row(grad_bits[t], topk_weights[t, j]))
            r = lay.slot[t, j]
            data[r], scales[r] = d, s
    return RecvBuffer(mode, H, lay.num_rows, data, scales, None)
