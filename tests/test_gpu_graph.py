"""HIP-graph capture of the whole path.

layout -> dispatch -> combine (layout and dispatch as two calls, or as the
one call ep_layout_dispatch) is captured once into a graph and replayed
several times; between replays the test does its own eager work (another
layout on other inputs, fills of the output buffers and of the workspace)
and synchronises, and it
checks every replay against the eager run of the same inputs.  The path
records no memset nodes (its kernels write every output they own).
"""

import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from tests.hip_path import DEV, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "layout_dispatch"])
@pytest.mark.parametrize("name", ["decode", "decode8", "small"])
def test_graph_replays_match_eager(ep, name, fused):
    print(f"\n[case] graph replay {name} fused={fused}", flush=True)
    sys.stdout.flush()
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w)
    idx, x, wts = to_dev(inp["topk_idx"]), to_dev(inp["x"]), to_dev(inp["topk_weights"])
    ws = torch.empty(ep.ep_workspace_bytes(w.t_max, w.k, w.E), dtype=torch.uint8, device=DEV)
    rc = torch.empty(w.E, dtype=torch.int64, device=DEV)
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    recv = torch.zeros(total, dtype=torch.uint8, device=DEV)
    y = to_dev(W.make_expert_out(w)).view(torch.uint8).reshape(-1) if w.combine_input == "normal" else None
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)

    def path():
        if fused:
            h = ep.ep_layout_dispatch(idx, w.E, w.t_max, rc, ws, x, w.H, w.mode, recv)
        else:
            h = ep.ep_layout(idx, w.E, w.t_max, rc, ws)
            ep.ep_dispatch(h, x, w.H, w.mode, recv)
        if y is None:
            ep.ep_combine(h, recv, w.mode if w.combine_input == "identity" else "none", w.H, idx, wts, out)
        else:
            ep.ep_combine(h, y, "none", w.H, idx, wts, out)
        return h

    h = path()
    torch.cuda.synchronize()
    R = int(rc.sum().item())
    slot_ptr = h.slot - ws.data_ptr()
    ref = dict(rc=rc.clone(), out=out.clone(), ws=ws[slot_ptr: slot_ptr + 4 * w.T * w.k].clone())
    dq, sq = {"none": (2 * w.H, 0), "int8_token": (w.H, 4), "fp8_b128": (w.H, w.H // 32)}[w.mode]
    ref_rows = recv[: R * dq].clone()

    # the "scaled_dispatch" workload's expert step is outside the path: combine
    # reads the receive buffer as bf16 here, in eager and graph runs alike
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    torch.cuda.synchronize()

    other = W.make_inputs(W.random_workload(77, 64, 64, w.E, w.k, "none"))
    idx2 = to_dev(other["topk_idx"])
    ws2 = torch.empty(ep.ep_workspace_bytes(64, w.k, w.E), dtype=torch.uint8, device=DEV)
    rc2 = torch.empty(w.E, dtype=torch.int64, device=DEV)
    for rep in range(4):
        out.fill_(float("nan"))
        rc.fill_(-1)
        recv.fill_(0xAB)
        ws.fill_(0xA5)                                 # every replay must write the layout again
        ep.ep_layout(idx2, w.E, 64, rc2, ws2)          # unrelated eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rc, ref["rc"]), f"replay {rep}: counts"
        assert torch.equal(ws[slot_ptr: slot_ptr + 4 * w.T * w.k], ref["ws"]), f"replay {rep}: slots"
        assert torch.equal(recv[: R * dq], ref_rows), f"replay {rep}: receive rows"
        assert torch.equal(out.view(torch.int16), ref["out"].view(torch.int16)), f"replay {rep}: combine"


@pytest.mark.parametrize("T", [16384, 33024], ids=["64chunks_two_launches", "129chunks_column_scan"])
def test_graph_replays_multichunk_layout(ep, T):
    """The multi-chunk layout (rank, then finalize; above 128 chunks with the
    column scan between them, which rewrites the chunk-count table in place)
    captured once and replayed over a workspace filled with garbage before
    every replay: each replay must give the eager counts, offsets, slots and
    row sources."""
    print(f"\n[case] graph replay layout T={T} k=8 E=256", flush=True)
    sys.stdout.flush()
    w = W.Workload("gl", T, 32, 256, 8, "int64", "none", "zipf", neg_frac=0.05, seed=9300 + T)
    inp = W.make_inputs(w)
    idx = to_dev(inp["topk_idx"])
    ws = torch.empty(ep.ep_workspace_bytes(w.t_max, w.k, w.E), dtype=torch.uint8, device=DEV)
    rc = torch.empty(w.E, dtype=torch.int64, device=DEV)
    ws.fill_(0xA5)
    h = ep.ep_layout(idx, w.E, w.t_max, rc, ws)
    torch.cuda.synchronize()
    off = lambda p: p - ws.data_ptr()
    views = [(off(h.offsets), 4 * (w.E + 1)), (off(h.slot), 4 * w.T * w.k), (off(h.row_src), 4 * w.max_rows)]
    ref_rc = rc.clone()
    ref = [ws[o: o + n].clone() for o, n in views]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ep.ep_layout(idx, w.E, w.t_max, rc, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        ws.fill_(0x5A + rep)
        rc.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rc, ref_rc), f"replay {rep}: counts"
        for (o, n), r in zip(views, ref):
            assert torch.equal(ws[o: o + n], r), f"replay {rep}: layout bytes at {o}"
