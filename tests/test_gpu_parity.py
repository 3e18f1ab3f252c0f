"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bars: layout (counts, offsets, slots, row sources, status) and quantised
codes/scales bit-exact; combine within 1 bf16 ulp of the oracle when the
combine input is bf16 and within 2e-2 relative error (per-row L2) when it is
quantised -- and, because both sides perform the same float32 operations in
the same order, also bit-exact, which is checked separately.

Every workload is compared in full, the 4096- and 16384-token ones at full
size and in the launch configuration the benchmark uses: the whole layout,
every routed receive row (the oracle's row quantiser, about 10 ms per
7168-wide row, runs in worker processes: tests/oracle_pool.py) and every
token of combine.
"""

import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import codecs, combine as C, layout as OL, quant as Q
from tests.hip_path import run_path, recv_rows
from tests.oracle_pool import dispatch_parallel
from tests.oracle_path import oracle_combine_bf16_rows, oracle_run

pytestmark = pytest.mark.gpu

SMALL = ["small", "decode8", "a5fused", "decode"]
LARGE = ["prefill", "large"]


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep      # raises if libep.so is missing
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _expert_out(w):
    return W.make_expert_out(w) if w.combine_input == "normal" else None


def _ulp_bf16(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -133)))
    return np.exp2(np.maximum(e, -126) - 7)


def check_combine(w, got_bits, want_bits):
    got = codecs.bf16_bits_to_f32(got_bits).astype(np.float64)
    want = codecs.bf16_bits_to_f32(want_bits).astype(np.float64)
    assert not (np.isnan(got) & ~np.isnan(want)).any(), "NaN in combine output (stray read of an unused row?)"
    # a dequantised value past float32's range is +-inf on both sides (IEEE);
    # those elements must match exactly, the tolerances apply to the rest
    fin = np.isfinite(want)
    assert np.array_equal(got_bits[~fin], want_bits[~fin])
    if w.combine_input == "identity" and w.mode != "none":
        rows = fin.all(axis=1)
        num = np.linalg.norm(got[rows] - want[rows], axis=1)
        den = np.maximum(np.linalg.norm(want[rows], axis=1), 1e-30)
        assert np.all(num / den <= 2e-2)
    else:
        assert np.all(np.abs(got[fin] - want[fin]) <= _ulp_bf16(want[fin]))
    # same float32 operations in the same order: expect identical bits
    assert np.array_equal(got_bits, want_bits)


def check_layout(run, lay):
    assert np.array_equal(run.recv_count, lay.count)
    assert np.array_equal(run.offsets, lay.offsets.astype(np.int32))
    assert np.array_equal(run.slot, lay.slot)
    assert np.array_equal(run.row_src, lay.row_src)
    assert run.status == lay.status


@pytest.mark.parametrize("name", SMALL)
def test_workload_full(ep, name):
    w = W.WORKLOADS[name]
    _announce(f"full parity {name} T={w.T} H={w.H} E={w.E} k={w.k} {w.mode}")
    inp = W.make_inputs(w)
    y = _expert_out(w)
    run = run_path(ep, w, inp, expert_out=y)
    lay, rb, out = oracle_run(w, inp, y)
    check_layout(run, lay)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R])
    assert np.array_equal(scales[:R], rb.scales[:R])
    assert np.array_equal(run.recv_weights[:R].cpu().numpy(), rb.weights[:R])
    check_combine(w, run.out, out)


def full_size_expected(w, inp, y):
    """The oracle's layout, receive rows and combine output of a whole
    full-size workload (rows quantised in worker processes)."""
    lay = OL.layout(inp["topk_idx"], w.E, w.t_max, row_align=w.row_align, expert_capacity=w.expert_capacity)
    rb = dispatch_parallel(inp["x"], lay, w.mode)
    if w.combine_input == "normal":
        out = oracle_combine_bf16_rows(w, inp, lay, y)
    else:                                            # identity experts: combine reads the dispatched rows
        assert w.combine_input == "identity"
        out = C.combine(rb, lay, inp["topk_weights"])
    return lay, rb, out


@pytest.mark.parametrize("name", LARGE)
def test_workload_full_size(ep, name):
    w = W.WORKLOADS[name]
    _announce(f"full-size parity {name} T={w.T} H={w.H} E={w.E} k={w.k} {w.mode}")
    inp = W.make_inputs(w)
    y = _expert_out(w)
    run = run_path(ep, w, inp, expert_out=y)
    lay, rb, out = full_size_expected(w, inp, y)
    check_layout(run, lay)                          # whole layout, bit-exact
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R])    # every routed row
    assert np.array_equal(scales[:R], rb.scales[:R])
    check_combine(w, run.out, out)                  # every token
    if name == "prefill":                            # Zipf: hot experts hold > 10x the mean
        assert lay.count.max() > 10 * lay.count.mean()


def test_determinism(ep):
    w = W.WORKLOADS["decode"]
    _announce("determinism decode")
    inp = W.make_inputs(w)
    y = _expert_out(w)
    a = run_path(ep, w, inp, expert_out=y)
    b = run_path(ep, w, inp, expert_out=y)
    assert np.array_equal(a.slot, b.slot) and np.array_equal(a.out, b.out)
    R = int(a.offsets[-1])
    da, sa = recv_rows(ep, a, w)
    db, sb = recv_rows(ep, b, w)
    assert np.array_equal(da[:R], db[:R]) and np.array_equal(sa[:R], sb[:R])
