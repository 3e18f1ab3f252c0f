"""Test helpers: run the HIP library and the CPU oracle on the same seeded
inputs and read the HIP results back for comparison.

The HIP side goes only through the C ABI (``combine_topk_idx_amd.ep``); the
oracle side only through ``oracle``.  The two never exchange data: each one
builds its own combine input from its own dispatch output when the workload
feeds dispatched rows back into combine.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from combine_topk_idx_amd import workloads as W

NAN_BF16 = 0x7FC0
DEV = "cuda"


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class HipRun:
    handle: object
    workspace: torch.Tensor
    recv_count: np.ndarray
    offsets: np.ndarray
    slot: np.ndarray
    row_src: np.ndarray
    status: int
    recv: torch.Tensor            # uint8 receive buffer
    recv_weights: torch.Tensor | None
    out: np.ndarray | None        # uint16 [T, H]


def ws_view(ws: torch.Tensor, ptr: int, n: int, dtype) -> torch.Tensor:
    off = ptr - ws.data_ptr()
    item = torch.empty((), dtype=dtype).element_size()
    return ws[off: off + n * item].view(dtype)


def canary_buffer(total: int) -> torch.Tensor:
    """uint8 buffer whose every bf16 lane is a NaN canary (0x7FC0)."""
    b = torch.empty(max(total, 16) // 2 * 2 + 16, dtype=torch.uint8, device=DEV)
    b.view(torch.int16).fill_(NAN_BF16)
    return b


def run_layout(ep, w: W.Workload, idx: np.ndarray, cum=None):
    padded = w.row_align > 1 or w.expert_capacity > 0
    if padded:
        nbytes = ep.ep_workspace_bytes_ex(w.t_max, w.k, w.E, w.row_align, w.expert_capacity)
    else:
        nbytes = ep.ep_workspace_bytes(w.t_max, w.k, w.E)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)                                   # garbage: nothing may rely on zeroed workspace
    recv_count = torch.full((w.E,), -7, dtype=torch.int64, device=DEV)
    if padded:
        h = ep.ep_layout_ex(to_dev(idx), w.E, w.t_max, w.row_align, w.expert_capacity, recv_count, ws, cum)
    else:
        h = ep.ep_layout(to_dev(idx), w.E, w.t_max, recv_count, ws, cum)
    assert h.max_rows == w.max_rows
    return h, ws, recv_count


def read_layout(ep, h, ws, recv_count, w):
    torch.cuda.synchronize()
    return dict(
        recv_count=recv_count.cpu().numpy(),
        offsets=ws_view(ws, h.offsets, w.E + 1, torch.int32).cpu().numpy(),
        slot=ws_view(ws, h.slot, w.T * w.k, torch.int32).cpu().numpy().reshape(w.T, w.k),
        row_src=ws_view(ws, h.row_src, w.max_rows, torch.int32).cpu().numpy(),
        status=ep.ep_read_status(h),
    )


def run_layout_dispatch(ep, w: W.Workload, idx: np.ndarray, x, wts, recv, recv_w, cum=None):
    """ep_layout_dispatch (layout and dispatch in one call) on fresh,
    garbage-filled workspace and counts."""
    nbytes = ep.ep_workspace_bytes_ex(w.t_max, w.k, w.E, w.row_align, w.expert_capacity)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)
    recv_count = torch.full((w.E,), -7, dtype=torch.int64, device=DEV)
    h = ep.ep_layout_dispatch(to_dev(idx), w.E, w.t_max, recv_count, ws, x, w.H, w.mode, recv, wts, recv_w, cum,
                              row_align=w.row_align, expert_capacity=w.expert_capacity, interleaved=w.interleaved)
    assert h.max_rows == w.max_rows
    return h, ws, recv_count


def run_path(ep, w: W.Workload, inp: dict, *, expert_out: np.ndarray | None = None,
             with_recv_weights=True, do_combine=True, fused=False) -> HipRun:
    """layout -> dispatch -> (expert step) -> combine on the GPU (fused: the
    first two through ep_layout_dispatch)."""
    x = to_dev(inp["x"])
    wts = to_dev(inp["topk_weights"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode, w.interleaved)
    recv = canary_buffer(total)
    recv_w = torch.full((max(w.max_rows, 1),), float("nan"), device=DEV) if with_recv_weights else None
    if fused:
        h, ws, recv_count = run_layout_dispatch(ep, w, inp["topk_idx"], x, wts if with_recv_weights else None,
                                                recv, recv_w)
    else:
        h, ws, recv_count = run_layout(ep, w, inp["topk_idx"])
        ep.ep_dispatch(h, x, w.H, w.mode, recv, wts if with_recv_weights else None, recv_w,
                       interleaved=w.interleaved)
    lay = read_layout(ep, h, ws, recv_count, w)
    out = None
    if do_combine:
        il = False
        if w.combine_input == "identity":
            src, q, il = recv, w.mode, w.interleaved
        elif w.combine_input == "scaled_dispatch":
            assert w.mode == "none"
            rows = recv[: w.max_rows * w.H * 2].view(torch.bfloat16)
            src = canary_buffer(total)
            src[: w.max_rows * w.H * 2].view(torch.bfloat16).copy_((rows.float() * 1.5).to(torch.bfloat16))
            q = "none"
        else:
            assert expert_out is not None
            y = expert_out.copy()
            y[lay["row_src"] < 0] = NAN_BF16             # rows holding no pair: canaries
            src, q = to_dev(y).view(torch.uint8).reshape(-1), "none"
        o = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
        ep.ep_combine(h, src, q, w.H, to_dev(inp["topk_idx"]), wts, o, interleaved=il)
        torch.cuda.synchronize()
        out = bf16_bits(o)
        # the ids given to combine are dispatch's: the routing check must
        # leave the layout's status word as it was
        after = ep.ep_read_status(h)
        assert after == lay["status"], f"combine changed the status word {lay['status']:#x} -> {after:#x}"
    return HipRun(h, ws, lay["recv_count"], lay["offsets"], lay["slot"], lay["row_src"], lay["status"],
                  recv, recv_w, out)


def recv_rows(ep, run: HipRun, w: W.Workload, rows=None):
    """(data [n, Dq], scales [n, Sq]) of the HIP receive buffer (numpy)."""
    from oracle import quant as Q   # row sizes only
    dq, sq = Q.row_bytes(w.mode, w.H)
    total, off = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode, w.interleaved)
    buf = run.recv
    n = w.max_rows
    if w.interleaved:
        stride = total // max(w.max_rows, 1)
        rowsv = buf[: w.max_rows * stride].view(w.max_rows, stride)
        if rows is not None:
            rowsv = rowsv.index_select(0, torch.as_tensor(np.asarray(rows, np.int64), device=DEV))
            n = len(rows)
        r = rowsv.cpu().numpy()
        return r[:, :dq].copy(), r[:, off:off + sq].copy()
    data = buf[: w.max_rows * dq].view(w.max_rows, dq)
    if rows is not None:
        idx = torch.as_tensor(np.asarray(rows, np.int64), device=DEV)
        data = data.index_select(0, idx)
        n = len(rows)
    if not sq:
        return data.cpu().numpy(), np.zeros((n, 0), np.uint8)
    scales = buf[off: off + w.max_rows * sq].view(w.max_rows, sq)
    if rows is not None:
        scales = scales.index_select(0, idx)
    return data.cpu().numpy(), scales.cpu().numpy()


LAYOUT_CHUNK_PAIRS = 2048   # pairs per workgroup of the multi-workgroup layout


def sample_tokens(w: W.Workload, idx: np.ndarray, n: int = 640, seed: int = 0, window: int = 256,
                  hot_cap: int = 256) -> np.ndarray:
    """Tokens to compare at full size: the first and last 8, `n` random ones,
    every token of two `window`-token spans centred on boundaries between
    the layout's 2048-pair chunks (the middle one and the last one), and up
    to `hot_cap` tokens routed to the busiest expert (evenly spaced, its
    first and last included).  At 4096 tokens and more this is over 1024
    tokens."""
    rng = np.random.default_rng(seed)
    T = w.T
    picks = set(range(min(8, T))) | set(range(max(0, T - 8), T))
    picks |= set(rng.choice(T, size=min(n, T), replace=False).tolist())
    chunk_tokens = max(LAYOUT_CHUNK_PAIRS // max(w.k, 1), 1)
    nchunks = (T + chunk_tokens - 1) // chunk_tokens
    if nchunks > 1 and window > 0:
        for b in sorted({chunk_tokens * (nchunks // 2), chunk_tokens * (nchunks - 1)}):
            picks |= set(range(max(0, b - window // 2), min(T, b + window // 2)))
    flat = idx.reshape(-1)
    valid = flat[(flat >= 0) & (flat < w.E)]
    if valid.size and hot_cap > 0:
        hot = np.bincount(valid, minlength=w.E).argmax()
        hot_tok = np.nonzero((idx == hot).any(axis=1))[0]
        if hot_tok.size > hot_cap:
            hot_tok = hot_tok[np.unique(np.linspace(0, hot_tok.size - 1, hot_cap).round().astype(np.int64))]
        picks |= set(hot_tok.tolist())
    return np.array(sorted(picks), np.int64)
