"""GPU parity at the largest arguments the library takes: top-16 of 512
experts ("Low-Latency Mode API", Constraints; the library's k <= 16 and
E <= 512), with over two million (token, j) pairs, so the layout runs over
1024 chunks of 2048 pairs and every finalize workgroup sums a 1024 x 512
table of chunk counts.

* the layout alone at T = 131072 (2,097,152 pairs) in the compact, the
  widest aligned (1024 rows) and a capacity-padded arrangement (3600 rows
  per expert, below the demand of about half the experts (mean 3686): the
  overflow bit and the dropped pairs), against the oracle bit for bit;
* the whole path at T = 65536 (1,048,576 pairs) with the smallest hidden
  size (32), unquantised rows and bf16 expert outputs: every routed row and
  every token of combine against the oracle.
"""

import sys
from dataclasses import replace

import numpy as np
import pytest

from combine_topk_idx_amd import workloads as W
from oracle import layout as OL
from tests.hip_path import read_layout, recv_rows, run_layout, run_path
from tests.oracle_path import oracle_run
from tests.test_gpu_parity import check_combine, check_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


MAX_LAYOUT = W.Workload("max_layout", 131072, 32, 512, 16, "int32", "none", "uniform", neg_frac=0.1, seed=9101)


@pytest.mark.parametrize("align,cap", [(1, 0), (1024, 0), (1, 3600)], ids=["compact", "align1024", "cap3600"])
def test_layout_max_pairs(ep, align, cap):
    w = replace(MAX_LAYOUT, row_align=align, expert_capacity=cap)
    _announce(f"layout T={w.T} k={w.k} E={w.E} align={align} cap={cap} rows={w.max_rows}")
    inp = W.make_inputs(w)
    h, ws, rc = run_layout(ep, w, inp["topk_idx"])
    got = read_layout(ep, h, ws, rc, w)
    lay = OL.layout(inp["topk_idx"], w.E, w.t_max, row_align=align, expert_capacity=cap)
    assert np.array_equal(got["recv_count"], lay.count)
    assert np.array_equal(got["offsets"], lay.offsets.astype(np.int32))
    assert np.array_equal(got["slot"], lay.slot)
    assert np.array_equal(got["row_src"], lay.row_src)
    assert got["status"] == lay.status
    if cap:
        assert lay.status & 2 and (lay.slot < 0).sum() > (inp["topk_idx"] < 0).sum()


def test_path_max_topk_and_experts(ep):
    w = W.Workload("max_path", 65536, 32, 512, 16, "int64", "none", "uniform", neg_frac=0.1, seed=9102,
                   combine_input="normal")
    _announce(f"path T={w.T} k={w.k} E={w.E} H={w.H} {w.mode}")
    inp = W.make_inputs(w)
    y = W.make_expert_out(w)
    run = run_path(ep, w, inp, expert_out=y)
    lay, rb, out = oracle_run(w, inp, y)
    check_layout(run, lay)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R])
    assert np.array_equal(run.recv_weights[:R].cpu().numpy(), rb.weights[:R])
    check_combine(w, run.out, out)


@pytest.mark.parametrize("T,align,cap", [(32768, 1, 0), (33024, 1, 0), (33024, 256, 0), (40000, 1, 160)],
                         ids=["128chunks", "129chunks", "129chunks-align256", "157chunks-cap160"])
def test_layout_around_column_scan(ep, T, align, cap):
    """Both sides of the chunk count (128) above which the layout scans its
    count table in a kernel of its own: 262144 pairs (two launches) and
    264192 pairs (three), compact, aligned and overflowing capacity blocks,
    against the oracle bit for bit."""
    w = W.Workload("colscan", T, 32, 256, 8, "int64", "none", "zipf", neg_frac=0.05, seed=9200 + T,
                   row_align=align, expert_capacity=cap)
    _announce(f"layout T={w.T} k={w.k} E={w.E} align={align} cap={cap} ({w.T * w.k // 2048} chunks)")
    inp = W.make_inputs(w)
    h, ws, rc = run_layout(ep, w, inp["topk_idx"])
    got = read_layout(ep, h, ws, rc, w)
    lay = OL.layout(inp["topk_idx"], w.E, w.t_max, row_align=align, expert_capacity=cap)
    assert np.array_equal(got["recv_count"], lay.count)
    assert np.array_equal(got["offsets"], lay.offsets.astype(np.int32))
    assert np.array_equal(got["slot"], lay.slot)
    assert np.array_equal(got["row_src"], lay.row_src)
    assert got["status"] == lay.status
    if cap:
        assert lay.status & 2
