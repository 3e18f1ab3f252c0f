"""GPU: ep_layout_dispatch_noalloc (the layout + dispatch call that brings
its own static workspace and allocates nothing) against ep_layout_dispatch
with a caller workspace, through the C ABI, on two calls in a row, the
second with a smaller input: every output (receive buffer with the canaries
of unused rows, counts, running statistics, receive weights, status), the
layout arrays its handle points to and combine through either handle are
identical.  (A layout larger than the static workspace is refused before
anything is launched: ``tests/test_abi_host.py``.)"""

import ctypes
import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from tests.hip_path import DEV, bf16_bits, canary_buffer, to_dev

pytestmark = pytest.mark.gpu

_hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch has loaded (same soname)
_hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
_hip.hipMemcpy.restype = ctypes.c_int
HIP_D2H = 2


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _read(ptr: int, n: int, dtype) -> np.ndarray:
    """n elements at device address ptr (synchronous copy)."""
    out = np.empty(n, dtype)
    if n:
        assert _hip.hipMemcpy(out.ctypes.data, ptr, out.nbytes, HIP_D2H) == 0
    return out


def _layout_arrays(h, T, k, E):
    return {"offsets": _read(h.offsets, E + 1, np.int32), "slot": _read(h.slot, T * k, np.int32),
            "row_src": _read(h.row_src, h.max_rows, np.int32), "status_word": _read(h.status, 1, np.uint32)}


def _run(ep, w, inp, noalloc):
    idx, x, wts = to_dev(inp["topk_idx"]), to_dev(inp["x"]), to_dev(inp["topk_weights"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    recv = canary_buffer(total)
    recv_w = torch.full((w.max_rows,), float("nan"), device=DEV)
    rc = torch.full((w.E,), -7, dtype=torch.int64, device=DEV)
    cum = torch.full((w.E,), 5, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    if noalloc:
        h = ep.ep_layout_dispatch_noalloc(idx, w.E, w.t_max, rc, x, w.H, w.mode, recv, wts, recv_w, cum,
                                          row_align=w.row_align, expert_capacity=w.expert_capacity)
        ws = None
    else:
        nb = ep.ep_workspace_bytes_ex(w.t_max, w.k, w.E, w.row_align, w.expert_capacity)
        ws = torch.full((max(nb, 256),), 0xA5, dtype=torch.uint8, device=DEV)
        h = ep.ep_layout_dispatch(idx, w.E, w.t_max, rc, ws, x, w.H, w.mode, recv, wts, recv_w, cum,
                                  row_align=w.row_align, expert_capacity=w.expert_capacity)
    torch.cuda.synchronize()
    lay = _layout_arrays(h, w.T, w.k, w.E)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.ep_combine(h, recv, w.mode, w.H, idx, wts, out)
    torch.cuda.synchronize()
    return dict(recv=recv.cpu().numpy(), recv_w=recv_w.cpu().numpy(), rc=rc.cpu().numpy(), cum=cum.cpu().numpy(),
                out=bf16_bits(out), status=ep.ep_read_status(h), **lay), ws


CALLS = [
    # the decode workload (one launch), then a smaller one (fewer tokens,
    # experts and rows), then capacity blocks that overflow (one launch), then
    # aligned blocks (two launches)
    W.replace(W.WORKLOADS["decode"], combine_input="identity"),
    W.Workload("smaller", 40, 1024, 16, 4, "int32", "mxfp8", "uniform", neg_frac=0.1, combine_input="identity",
               seed=3301),
    W.Workload("capacity", 60, 512, 8, 4, "int64", "fp8_b128", "uniform", neg_frac=0.05, combine_input="identity",
               seed=3303, expert_capacity=20),
    W.Workload("aligned", 30, 512, 8, 2, "int64", "mxfp4", "uniform", combine_input="identity", seed=3302,
               num_max_tokens=33, row_align=32),
]


def test_noalloc_matches_layout_dispatch(ep):
    print("\n[case] ep_layout_dispatch_noalloc vs ep_layout_dispatch, four calls in a row", flush=True)
    sys.stdout.flush()
    for w in CALLS:
        inp = W.make_inputs(w)
        a, _ = _run(ep, w, inp, noalloc=True)
        b, ws = _run(ep, w, inp, noalloc=False)
        for key in a:
            x, y = np.asarray(a[key]), np.asarray(b[key])
            assert np.array_equal(x, y, equal_nan=x.dtype.kind == "f"), f"{w.name}: {key} differs"
        print(f"{w.name}: T={w.T} rows={w.max_rows} identical", flush=True)
