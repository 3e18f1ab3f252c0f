"""Dispatch of the oracle (test infrastructure only).

Each token row is quantised once ("Low-Latency Mode API", Parameters
``use_fp8`` / ``use_ue8m0`` / ``use_mxfp4``; "DeepEP FP8 Dispatch and Combine
Operations", "The Dispatch Stage") and copied to the receive row
``slot[t, j]`` of every routed pair.

Receive buffer ("EP dispatch with unfused MXFP8 quantization", Changes: data
and block scales share one caller buffer, sliced into a data region followed
by a scale region; the pages do not fix the exact layout, so this is the
reading taken -- compact expert-major rows, row-major scales):

* data region: ``max_rows`` rows of ``Dq`` bytes, row-major;
* scale region: starts at ``align_up(max_rows * Dq, 256)``; ``max_rows`` rows
  of ``Sq`` bytes.  bf16 rows have no scale region and no padding.

``Dq``/``Sq`` per mode are in ``quant.row_bytes``.  Rows at or past R and the
padding between the regions are unspecified and never compared.

If ``topk_weights`` is given, ``recv_weights[slot[t, j]] = topk_weights[t, j]``
(the pages list the argument without saying what dispatch does with it;
this is the reading taken).

Parity: the ``none`` mode is pinned by ``recv[slot[t, j]] == x[t]`` bit for
bit; the quantised modes inherit the pins of ``quant``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import quant
from .layout import Layout

SCALE_REGION_ALIGN = 256


def align_up(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def buffer_bytes(rows: int, hidden: int, mode: str) -> tuple[int, int]:
    """(total bytes, scale-region offset) of a receive buffer of ``rows``."""
    dq, sq = quant.row_bytes(mode, hidden)
    off = align_up(rows * dq, SCALE_REGION_ALIGN) if sq else rows * dq
    return off + rows * sq, off


@dataclass
class RecvBuffer:
    mode: str
    hidden: int
    num_rows: int                # R: rows [0, R) are defined
    data: np.ndarray             # uint8 [max_rows, Dq]
    scales: np.ndarray           # uint8 [max_rows, Sq]
    weights: np.ndarray | None   # float32 [max_rows] or None

    def to_bytes(self) -> np.ndarray:
        """The flat buffer: data region, zero padding, scale region."""
        rows = self.data.shape[0]
        total, off = buffer_bytes(rows, self.hidden, self.mode)
        buf = np.zeros(total, np.uint8)
        buf[:self.data.size] = self.data.reshape(-1)
        buf[off:off + self.scales.size] = self.scales.reshape(-1)
        return buf

    @staticmethod
    def from_bytes(buf: np.ndarray, rows: int, hidden: int, mode: str, num_rows: int) -> "RecvBuffer":
        dq, sq = quant.row_bytes(mode, hidden)
        total, off = buffer_bytes(rows, hidden, mode)
        buf = np.asarray(buf, np.uint8).reshape(-1)
        if buf.size < total:
            raise ValueError("buffer too small")
        data = buf[:rows * dq].reshape(rows, dq)
        scales = buf[off:off + rows * sq].reshape(rows, sq)
        return RecvBuffer(mode, hidden, num_rows, data, scales, None)


def dispatch(x_bits: np.ndarray, lay: Layout, mode: str,
             topk_weights: np.ndarray | None = None) -> RecvBuffer:
    """x_bits: uint16 [T, H] bf16 patterns.  Returns the receive buffer."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    if T != lay.num_tokens:
        raise ValueError("x and layout disagree on num_tokens")
    dq, sq = quant.row_bytes(mode, H)
    data = np.zeros((lay.max_rows, dq), np.uint8)
    scales = np.zeros((lay.max_rows, sq), np.uint8)
    weights = None
    if topk_weights is not None:
        weights = np.zeros(lay.max_rows, np.float32)
    for t in range(T):
        routed = [j for j in range(lay.num_topk) if lay.slot[t, j] >= 0]
        if not routed:
            continue
        d, s = quant.quantize_row(mode, x_bits[t])
        for j in routed:
            r = lay.slot[t, j]
            data[r] = d
            scales[r] = s
            if weights is not None:
                weights[r] = topk_weights[t, j]
    return RecvBuffer(mode, H, lay.num_rows, data, scales, weights)


def dispatch_tokens(x_bits: np.ndarray, lay: Layout, mode: str, tokens) -> dict:
    """The packed rows of a sample of tokens only: {row: (data, scales)} for
    every routed pair of the listed tokens.  Used to check full-size runs
    one token at a time."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    out = {}
    for t in tokens:
        t = int(t)
        rows = [int(lay.slot[t, j]) for j in range(lay.num_topk) if lay.slot[t, j] >= 0]
        if not rows:
            continue
        d, s = quant.quantize_row(mode, x_bits[t])
        for r in rows:
            out[r] = (d, s)
    return out
