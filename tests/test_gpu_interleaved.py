"""GPU parity of the interleaved receive form (EP_RECV_INTERLEAVED: every row
holds its data, then its scales) against the oracle's serialisation of the
same rows: dispatch, combine from interleaved rows and the combine backward.

Bars: every byte of every row that holds a pair (data, scales and the row's
padding up to the next 16-byte row start, which the oracle leaves zero and
the kernels never write -- so the padding is only checked to be untouched
canary bytes) equal to the oracle's; combine output bit-exact.
"""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import backward as OB, dispatch as OD, layout as OL, quant as OQ
from tests.hip_path import canary_buffer, recv_rows, run_layout, run_path, to_dev
from tests.oracle_path import oracle_run
from tests.test_gpu_parity import check_combine, check_layout, full_size_expected

pytestmark = pytest.mark.gpu

MODES = ["int8_token", "fp8_b128", "mxfp8", "mxfp4", "fp8_b128_pow2", "fp8_b128_ue8m0"]


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("H", [384, 7168])
def test_interleaved_dispatch_combine(ep, mode, H):
    w = W.Workload("il", 40, H, 16, 4, "int64", mode, "uniform", neg_frac=0.1, combine_input="identity",
                   seed=8100 + H, interleaved=True)
    _announce(f"interleaved {mode} H={H}")
    inp = W.make_inputs(w)
    run = run_path(ep, w, inp)
    lay, rb, out = oracle_run(w, inp)
    check_layout(run, lay)
    rows = lay.valid_rows()
    # whole rows of the raw buffer against the oracle's interleaved bytes
    want = rb.to_bytes(interleaved=True)
    stride = OD.interleaved_stride(H, mode)
    dq, sq = OQ.row_bytes(mode, H)
    got = run.recv[: w.max_rows * stride].view(w.max_rows, stride).cpu().numpy()
    want = want.reshape(w.max_rows, stride)
    assert np.array_equal(got[rows, : dq + sq], want[rows, : dq + sq])
    pad = got[rows, dq + sq:]
    canary = np.frombuffer(np.full(stride, 0x7FC0, np.uint16).tobytes(), np.uint8)[dq + sq: stride]
    assert np.array_equal(pad, np.broadcast_to(canary, pad.shape))      # padding never written
    check_combine(w, run.out, out)


def test_interleaved_matches_region_form_combine(ep):
    """The same dispatch into both forms: identical rows, identical combine."""
    base = replace(W.WORKLOADS["decode"], mode="mxfp8", combine_input="identity")
    _announce("interleaved vs region form, decode shape")
    inp = W.make_inputs(base)
    a = run_path(ep, base, inp)
    b = run_path(ep, replace(base, interleaved=True), inp)
    assert np.array_equal(a.out, b.out)
    da, sa = recv_rows(ep, a, base)
    db, sb = recv_rows(ep, b, replace(base, interleaved=True))
    rows = np.nonzero(a.row_src >= 0)[0]
    assert np.array_equal(da[rows], db[rows]) and np.array_equal(sa[rows], sb[rows])


def test_interleaved_full_size(ep):
    """The prefill workload in the interleaved form at full size: the whole
    layout, every routed row and every token of combine."""
    w = replace(W.WORKLOADS["prefill"], interleaved=True)
    _announce(f"interleaved full-size prefill {w.mode}")
    inp = W.make_inputs(w)
    run = run_path(ep, w, inp)
    lay, rb, out = full_size_expected(w, inp, None)
    check_layout(run, lay)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R]) and np.array_equal(scales[:R], rb.scales[:R])
    check_combine(w, run.out, out)


@pytest.mark.parametrize("mode", ["mxfp8", "fp8_b128_ue8m0", "int8_token"])
def test_interleaved_backward(ep, mode):
    T, H, E, k = 30, 512, 16, 8
    w = W.Workload("ilb", T, H, E, k, "int64", mode, "uniform", neg_frac=0.1, seed=8300, interleaved=True)
    _announce(f"interleaved backward {mode}")
    inp = W.make_inputs(w)
    grad = W.make_inputs(W.Workload("g", T, H, E, k, "int64", mode, "uniform", seed=8301))["x"]
    h, ws, rc = run_layout(ep, w, inp["topk_idx"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, H, mode, True)
    buf = canary_buffer(total)
    ep.ep_combine_backward(h, to_dev(grad), H, mode, buf, to_dev(inp["topk_weights"]), interleaved=True)
    torch.cuda.synchronize()
    lay = OL.layout(inp["topk_idx"], E, T)
    rb = OB.combine_backward(grad, lay, mode, inp["topk_weights"])
    stride = OD.interleaved_stride(H, mode)
    dq, sq = OQ.row_bytes(mode, H)
    got = buf[: w.max_rows * stride].view(w.max_rows, stride).cpu().numpy()
    want = rb.to_bytes(interleaved=True).reshape(w.max_rows, stride)
    rows = lay.valid_rows()
    assert np.array_equal(got[rows, : dq + sq], want[rows, : dq + sq])
