"""Test helper: the oracle's run of a whole workload (layout -> dispatch ->
expert step -> combine), optionally restricted to a sample of tokens."""

from __future__ import annotations

import numpy as np

from combine_topk_idx_amd import workloads as W
from oracle import combine as C, dispatch as D, layout as L, quant as Q


def oracle_run(w: W.Workload, inp: dict, expert_out: np.ndarray | None = None, tokens=None):
    lay = L.layout(inp["topk_idx"], w.E, w.t_max, row_align=w.row_align, expert_capacity=w.expert_capacity)
    dq, sq = Q.row_bytes(w.mode, w.H)
    if tokens is None:
        rb = D.dispatch(inp["x"], lay, w.mode, inp["topk_weights"])
    else:
        rows = D.dispatch_tokens(inp["x"], lay, w.mode, tokens)
        data = np.zeros((w.max_rows, dq), np.uint8)
        scales = np.zeros((w.max_rows, sq), np.uint8)
        for r, (d, s) in rows.items():
            data[r], scales[r] = d, s
        rb = D.RecvBuffer(w.mode, w.H, lay.num_rows, data, scales, None)
    if w.combine_input == "identity":
        cin = rb
    elif w.combine_input == "scaled_dispatch":
        from oracle import codecs
        y = codecs.bf16_bits_to_f32(rb.data.view(np.uint16)).astype(np.float32) * np.float32(1.5)
        cin = D.RecvBuffer("none", w.H, lay.num_rows, W.bf16_from_f32(y).view(np.uint8),
                           np.zeros((w.max_rows, 0), np.uint8), None)
    else:
        cin = D.RecvBuffer("none", w.H, lay.num_rows, expert_out.view(np.uint8).reshape(w.max_rows, -1),
                           np.zeros((w.max_rows, 0), np.uint8), None)
    out = C.combine(cin, lay, inp["topk_weights"], tokens)
    return lay, rb, out


def oracle_combine_bf16_rows(w: W.Workload, inp: dict, lay, expert_out: np.ndarray, tokens=None) -> np.ndarray:
    """The oracle's combine of bf16 expert rows (a workload whose combine
    input does not depend on the dispatched rows), for every token or a
    sample; the rows are read as they are, so no dispatch is needed."""
    cin = D.RecvBuffer("none", w.H, lay.num_rows, expert_out.view(np.uint8).reshape(w.max_rows, -1),
                       np.zeros((w.max_rows, 0), np.uint8), None)
    return C.combine(cin, lay, inp["topk_weights"], tokens)
