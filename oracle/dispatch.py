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

``Dq``/``Sq`` per mode are in ``quant.row_bytes``.  Rows that hold no pair and
the padding between the regions are unspecified and never compared.

Interleaved form ("DeepEP FP8 Dispatch and Combine Operations", Message
Transmission via IBGDA: each token's message is its FP8 payload followed by
its scales): row r starts at ``r * stride`` with ``stride = align_up(Dq + Sq,
128)``; its Dq data bytes come first, then its Sq scale bytes, then zero
padding.  The pages fix no alignment; every row starting on a 128-byte cache
line is the reading taken (rows that share lines cost the scattered writes
and gathers of the path a fifth to a third of their speed on MI355X).

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


INTERLEAVED_ROW_ALIGN = 128


def interleaved_stride(hidden: int, mode: str) -> int:
    dq, sq = quant.row_bytes(mode, hidden)
    return align_up(dq + sq, INTERLEAVED_ROW_ALIGN)


def buffer_bytes(rows: int, hidden: int, mode: str, interleaved: bool = False) -> tuple[int, int]:
    """(total bytes, scale offset) of a receive buffer of ``rows``: the
    scale-region offset, or for the interleaved form the offset of the
    scales inside a row."""
    dq, sq = quant.row_bytes(mode, hidden)
    if interleaved:
        return rows * interleaved_stride(hidden, mode), dq
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

    def to_bytes(self, interleaved: bool = False) -> np.ndarray:
        """The flat buffer: data region, zero padding, scale region; or, in
        the interleaved form, one row after another, each data then scales
        then zero padding."""
        rows, dq = self.data.shape
        sq = self.scales.shape[1]
        total, off = buffer_bytes(rows, self.hidden, self.mode, interleaved)
        buf = np.zeros(total, np.uint8)
        if interleaved:
            stride = interleaved_stride(self.hidden, self.mode)
            for r in range(rows):
                buf[r * stride:r * stride + dq] = self.data[r]
                buf[r * stride + dq:r * stride + dq + sq] = self.scales[r]
            return buf
        buf[:self.data.size] = self.data.reshape(-1)
        buf[off:off + self.scales.size] = self.scales.reshape(-1)
        return buf

    @staticmethod
    def from_bytes(buf: np.ndarray, rows: int, hidden: int, mode: str, num_rows: int,
                   interleaved: bool = False) -> "RecvBuffer":
        dq, sq = quant.row_bytes(mode, hidden)
        total, off = buffer_bytes(rows, hidden, mode, interleaved)
        buf = np.asarray(buf, np.uint8).reshape(-1)
        if buf.size < total:
            raise ValueError("buffer too small")
        if interleaved:
            stride = interleaved_stride(hidden, mode)
            rowsv = buf[:rows * stride].reshape(rows, stride)
            return RecvBuffer(mode, hidden, num_rows, rowsv[:, :dq].copy(), rowsv[:, dq:dq + sq].copy(), None)
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
