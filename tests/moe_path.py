"""Test helpers for the expert MLP: the GPU path through the C ABI and the
oracle path, on the same seeded inputs; neither side sees the other's data."""

from __future__ import annotations

import numpy as np
import torch

from combine_topk_idx_amd import workloads as W
from oracle import combine as OC, dispatch as OD, layout as OL, moe as OM
from tests.hip_path import DEV, canary_buffer, ws_view, to_dev, bf16_bits


def gpu_moe(ep, w: W.MoeWorkload, inp: dict, *, out_quant="mxfp8", pass_count=True, row_align=1,
            expert_capacity=0, stop_after=None):
    """layout -> dispatch (MXFP8) -> GMM1 (+SwiGLU, out_quant) -> GMM2 -> combine."""
    E = w.E_local
    padded = row_align > 1 or expert_capacity > 0
    if padded:
        wsb = ep.ep_workspace_bytes_ex(w.T, w.k, E, row_align, expert_capacity)
    else:
        wsb = ep.ep_workspace_bytes(w.T, w.k, E)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    rc = torch.empty(E, dtype=torch.int64, device=DEV)
    idx = to_dev(inp["topk_idx"])
    if padded:
        h = ep.ep_layout_ex(idx, E, w.T, row_align, expert_capacity, rc, ws)
    else:
        h = ep.ep_layout(idx, E, w.T, rc, ws)
    rows = h.max_rows
    xb, _ = ep.ep_buffer_bytes(rows, w.H, "mxfp8")
    recv = canary_buffer(xb)
    ep.ep_dispatch(h, to_dev(inp["x"]), w.H, "mxfp8", recv)
    w1c, w1s = ep.pack_moe_weights(to_dev(inp["w1_codes"]), to_dev(inp["w1_scales"]), True)
    w2c, w2s = ep.pack_moe_weights(to_dev(inp["w2_codes"]), to_dev(inp["w2_scales"]), False)
    ab, _ = ep.ep_buffer_bytes(rows, w.I, out_quant)
    a = canary_buffer(ab)
    ep.ep_moe_gmm1(h, recv, w.H, w.I, w1c, w1s, out_quant, a, recv_count=rc if pass_count else None)
    res = {"handle": h, "ws": ws, "rc": rc, "recv": recv, "a": a, "w2": (w2c, w2s)}
    if stop_after == "gmm1":
        torch.cuda.synchronize()
        return res
    y = canary_buffer(rows * w.H * 2)
    ep.ep_moe_gmm2(h, a, w.I, w.H, w2c, w2s, y, recv_count=rc if pass_count else None)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.ep_combine(h, y, "none", w.H, idx, to_dev(inp["topk_weights"]), out)
    torch.cuda.synchronize()
    res.update(y=y, out=bf16_bits(out))
    return res


def read_slots(ep, res, w):
    h = res["handle"]
    slot = ws_view(res["ws"], h.slot, w.T * w.k, torch.int32).cpu().numpy().reshape(w.T, w.k)
    offs = ws_view(res["ws"], h.offsets, w.E_local + 1, torch.int32).cpu().numpy()
    return slot, offs


def oracle_moe(w: W.MoeWorkload, inp: dict, *, out_mode="mxfp8", tokens=None, row_align=1, expert_capacity=0,
               parallel=False):
    """Oracle run; with `tokens`, only the rows of those tokens go through the
    MLP and only their combine rows are returned.  parallel: the dispatch's
    row quantiser runs in worker processes (tests/oracle_pool.py, the same
    rows as the oracle's dispatch) -- for full-size inputs."""
    lay = OL.layout(inp["topk_idx"], w.E_local, w.T, row_align=row_align, expert_capacity=expert_capacity)
    if parallel:
        from tests.oracle_pool import dispatch_parallel
        rb = dispatch_parallel(inp["x"], lay, "mxfp8")
    else:
        rb = OD.dispatch(inp["x"], lay, "mxfp8")
    want_rows = None
    if tokens is not None:
        want_rows = {int(r) for t in tokens for r in lay.slot[t] if r >= 0}
    per_expert = []
    y_rows = np.zeros((lay.max_rows, w.H), np.uint16)
    for e in range(w.E_local):
        r0, n = int(lay.offsets[e]), int(lay.count[e])
        rows = np.arange(r0, r0 + n)
        if want_rows is not None:
            rows = np.array(sorted(r for r in rows if r in want_rows), np.int64)
        if rows.size == 0:
            per_expert.append((rows, None))
            continue
        q, qs, a = OM.gmm1_swiglu_rows(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e],
                                       out_mode)
        entry = {"q": q, "qs": qs, "a": a}
        if out_mode == "mxfp8":
            yb, y = OM.gmm2_rows(q, qs, inp["w2_codes"][e], inp["w2_scales"][e])
            y_rows[rows] = yb
            entry["y"] = y
        per_expert.append((rows, entry))
    out = None
    if out_mode == "mxfp8":
        cin = OD.RecvBuffer("none", w.H, lay.num_rows, y_rows.view(np.uint8), np.zeros((lay.max_rows, 0), np.uint8),
                            None)
        out = OC.combine(cin, lay, inp["topk_weights"], tokens)
    return lay, rb, per_expert, out
