"""Pins of the oracle's combine backward (reverse dispatch).

* unit weights give exactly the unweighted rows (bf16(1 * g) == g);
* bf16 rows equal torch's float32 product rounded by torch's bf16 cast;
* the adjoint identity: for bf16 rows y and gradient g,
  sum_t <g[t], out[t]> == sum_r <dy[r], y[r]> where out = sum_j w y_j, up to
  the bf16 rounding of dy -- a misrouted row or a weight taken from the
  wrong j breaks it (planted below).
"""

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import backward as B, codecs, dispatch as D, layout as L


def _case(seed, T=30, H=64, E=6, k=4, neg=0.2):
    w = W.random_workload(seed, T, H, E, k, "none", neg_frac=neg)
    inp = W.make_inputs(w)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    return w, inp, lay


@pytest.mark.parametrize("mode", ["none", "int8_token", "mxfp8", "mxfp4"])
def test_unit_weights_equal_unweighted(mode):
    w, inp, lay = _case(1, H=128)
    a = B.combine_backward(inp["x"], lay, mode, np.ones((w.T, w.k), np.float32))
    b = B.combine_backward(inp["x"], lay, mode, None)
    R = lay.num_rows
    assert np.array_equal(a.data[:R], b.data[:R]) and np.array_equal(a.scales[:R], b.scales[:R])


def test_unweighted_is_dispatch_of_grad():
    w, inp, lay = _case(2)
    a = B.combine_backward(inp["x"], lay, "mxfp8", None)
    for t in range(w.T):
        for j in range(w.k):
            r = lay.slot[t, j]
            if r >= 0:
                from oracle import quant as Q
                d, s = Q.quantize_row("mxfp8", inp["x"][t])
                assert np.array_equal(a.data[r], d) and np.array_equal(a.scales[r], s)


def test_bf16_rows_match_torch():
    w, inp, lay = _case(3)
    rb = B.combine_backward(inp["x"], lay, "none", inp["topk_weights"])
    g = torch.from_numpy(codecs.bf16_bits_to_f32(inp["x"]).copy())
    for t in range(w.T):
        for j in range(w.k):
            r = lay.slot[t, j]
            if r < 0:
                continue
            want = (torch.tensor(inp["topk_weights"][t, j], dtype=torch.float32) * g[t]).to(torch.bfloat16)
            assert np.array_equal(rb.data[r].view(np.uint16), want.view(torch.int16).numpy().view(np.uint16))


def _adjoint_gap(inp, lay, rows_dy, w, wts):
    """|sum_t <g, out> - sum_r <dy, y>| relative to the magnitude."""
    y = W.make_expert_out(w)
    yf = codecs.bf16_bits_to_f32(y).astype(np.float64)
    g = codecs.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    lhs = mag = 0.0
    for t in range(w.T):
        out = np.zeros(w.H)
        for j in range(w.k):
            r = lay.slot[t, j]
            if r >= 0:
                out += float(wts[t, j]) * yf[r]
        lhs += float(g[t] @ out)
        mag += float(np.abs(g[t]) @ np.abs(out))
    dy = codecs.bf16_bits_to_f32(rows_dy.view(np.uint16)).astype(np.float64)
    rhs = sum(float(dy[r] @ yf[r]) for r in range(lay.num_rows))
    return abs(lhs - rhs) / max(mag, 1e-30)


@pytest.mark.parametrize("seed", range(3))
def test_adjoint_identity(seed):
    w, inp, lay = _case(10 + seed, T=40, H=96, E=5, k=6)
    wts = inp["topk_weights"]
    rb = B.combine_backward(inp["x"], lay, "none", wts)
    assert _adjoint_gap(inp, lay, rb.data, w, wts) <= 2.0 ** -8


def test_planted_wrong_weight_breaks_adjoint():
    w, inp, lay = _case(20, T=40, H=96, E=5, k=6)
    wts = inp["topk_weights"]
    shifted = np.roll(wts, 1, axis=1)                 # weight of another j
    rb = B.combine_backward(inp["x"], lay, "none", shifted)
    assert _adjoint_gap(inp, lay, rb.data, w, wts) > 2.0 ** -6


@pytest.mark.parametrize("weighted", [True, False])
def test_parallel_backward_helper_is_the_oracle_backward(weighted):
    """tests/oracle_pool.backward_parallel (the full-size GPU test's expected
    rows, quantised in worker processes) gives the oracle's combine backward
    row for row."""
    from tests.oracle_pool import backward_parallel
    w = W.random_workload(91, 200, 256, 16, 4, "mxfp8", neg_frac=0.2)
    inp = W.make_inputs(w)
    grad = W.make_inputs(W.random_workload(92, 200, 256, 16, 4, "mxfp8"))["x"]
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    wts = inp["topk_weights"] if weighted else None
    toks = list(range(0, 200, 3))
    want = B.combine_backward(grad, lay, "mxfp8", wts, tokens=toks)
    got = backward_parallel(grad, lay, "mxfp8", wts, toks, workers=2, chunk=17)
    rows = sorted({int(r) for t in toks for r in lay.slot[t] if r >= 0})
    assert sorted(got) == rows
    for r in rows:
        assert np.array_equal(got[r][0], want.data[r]) and np.array_equal(got[r][1], want.scales[r])
