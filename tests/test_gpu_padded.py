"""GPU parity of the aligned and capacity-padded receive arrangements
(``ep_layout_ex``) against the CPU oracle, on the same seeded inputs.

Bars as for the compact layout: the layout (counts, block starts, slots, row
sources including the -1 of every padding row, status bits) and every
quantised row that holds a pair are bit-exact; combine output bit-exact.
Padding rows of the receive and combine-input buffers hold NaN canaries, so a
read of a row that holds no pair shows up as NaN in the output.

Also checked: an arrangement without dropped pairs never changes combine's
result (the same float32 operations in the same order), and the
"Low-Latency Mode API" wrappers hand out [E, C, ...] views for a capacity C.
"""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import layout as OL
from tests.hip_path import run_path, recv_rows, to_dev, bf16_bits
from tests.oracle_path import oracle_run
from tests.test_gpu_parity import check_combine, check_layout, full_size_expected

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _expert_out(w):
    return W.make_expert_out(w) if w.combine_input == "normal" else None


# (workload, row_align, expert_capacity); capacity cases below the busiest
# expert's demand drop pairs and set the overflow bit
FULL = [
    ("small", 32, 0), ("small", 1, 20), ("small", 1, 64),
    ("decode8", 64, 0), ("decode8", 1, 192), ("decode8", 1, 150),
    ("a5fused", 1, 24),                        # every expert receives exactly 24
    ("decode", 16, 0), ("decode", 1, 4),
    ("decode", 1, 128),                        # capacity = num_max_dispatch_tokens
]


@pytest.mark.parametrize("name,align,cap", FULL)
def test_padded_full(ep, name, align, cap):
    w = replace(W.WORKLOADS[name], row_align=align, expert_capacity=cap)
    _announce(f"padded full {name} align={align} cap={cap} rows={w.max_rows} {w.mode}")
    inp = W.make_inputs(w)
    y = _expert_out(w)
    run = run_path(ep, w, inp, expert_out=y)
    lay, rb, out = oracle_run(w, inp, y)
    check_layout(run, lay)
    rows = lay.valid_rows()
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[rows], rb.data[rows])
    assert np.array_equal(scales[rows], rb.scales[rows])
    assert np.array_equal(run.recv_weights[rows].cpu().numpy(), rb.weights[rows])
    check_combine(w, run.out, out)
    if name == "a5fused":
        assert lay.count.tolist() == [24] * 8 and lay.status == 0
    demand = np.bincount(inp["topk_idx"][inp["topk_idx"] >= 0], minlength=w.E)
    assert bool(run.status & 2) == bool(cap and demand.max() > cap)


# full-size, multi-workgroup layout; the capacity case drops the Zipf
# routing's hot experts down to 4x the mean
FULL_SIZE = [("prefill", 128, 0), ("prefill", 1, 512), ("large", 64, 0)]


@pytest.mark.parametrize("name,align,cap", FULL_SIZE)
def test_padded_full_size(ep, name, align, cap):
    """Full size, multi-workgroup layout: the whole layout, every routed row
    (padding rows hold canaries the oracle does not define) and every token
    of combine."""
    w = replace(W.WORKLOADS[name], row_align=align, expert_capacity=cap, combine_input="identity")
    _announce(f"padded full-size {name} align={align} cap={cap} rows={w.max_rows} {w.mode}")
    inp = W.make_inputs(w)
    run = run_path(ep, w, inp)
    lay, rb, out = full_size_expected(w, inp, None)
    check_layout(run, lay)
    rows = np.nonzero(lay.row_src >= 0)[0]
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[rows], rb.data[rows])
    assert np.array_equal(scales[rows], rb.scales[rows])
    check_combine(w, run.out, out)
    if cap:
        assert run.status & 2 and lay.count.max() == cap


@pytest.mark.parametrize("name,align,cap", [("decode", 128, 0), ("decode", 1, 128), ("prefill", 256, 0)])
def test_arrangement_does_not_change_combine(ep, name, align, cap):
    base = replace(W.WORKLOADS[name], combine_input="identity")
    w = replace(base, row_align=align, expert_capacity=cap)
    _announce(f"arrangement invariance {name} align={align} cap={cap}")
    inp = W.make_inputs(base)
    a = run_path(ep, base, inp)
    b = run_path(ep, w, inp)
    assert b.status == 0
    assert np.array_equal(a.recv_count, b.recv_count)
    assert np.array_equal(a.out, b.out)
    # a pair's row moves from offsets[e] + i to the block start of e + i
    lay = OL.layout(inp["topk_idx"], w.E, w.t_max)
    flat = inp["topk_idx"].reshape(-1).astype(np.int64)
    ok = flat >= 0
    local = a.slot.reshape(-1)[ok] - a.offsets[flat[ok]]
    assert np.array_equal(b.slot.reshape(-1)[ok], b.offsets[flat[ok]] + local)
    assert np.all(b.offsets[:-1] % align == 0)
    assert lay.num_rows == int(a.offsets[-1])


def test_low_latency_capacity_views(ep):
    w = W.WORKLOADS["decode8"]
    _announce("low_latency capacity views decode8")
    inp = W.make_inputs(w)
    x = to_dev(inp["x"])
    idx = to_dev(inp["topk_idx"])
    wts = to_dev(inp["topk_weights"])
    C = w.T
    recv_x, cnt, h, _, _ = ep.low_latency_dispatch(x, idx, w.T, w.E, use_fp8=False, expert_capacity=C)
    assert tuple(recv_x.shape) == (w.E, C, w.H)
    out, _, _ = ep.low_latency_combine(recv_x, idx, wts, h)
    recv_c, cnt_c, h_c, _, _ = ep.low_latency_dispatch(x, idx, w.T, w.E, use_fp8=False)
    out_c, _, _ = ep.low_latency_combine(recv_c, idx, wts, h_c)
    torch.cuda.synchronize()
    assert torch.equal(cnt, cnt_c)
    assert np.array_equal(bf16_bits(out), bf16_bits(out_c))
    # expert e's first recv_count[e] rows are its tokens in order
    xs = inp["x"]
    e = 3
    toks = np.nonzero((inp["topk_idx"] == e).any(axis=1))[0]
    got = recv_x[e, : len(toks)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, xs[toks])
