"""GPU parity of ep_combine_backward (reverse dispatch of combine's gradient)
against the oracle: receive rows and scales bit-exact, with and without
weights, every mode, ragged shapes, and the large workload at full size on a
sample of tokens."""

import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import backward as OB, layout as OL
from tests.hip_path import DEV, canary_buffer, recv_rows, run_layout, sample_tokens, to_dev, HipRun
from tests.oracle_pool import backward_parallel, dispatch_parallel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _run(ep, w, inp, grad, weighted):
    h, ws, rc = run_layout(ep, w, inp["topk_idx"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    buf = canary_buffer(total)
    ep.ep_combine_backward(h, to_dev(grad), w.H, w.mode, buf,
                           to_dev(inp["topk_weights"]) if weighted else None)
    torch.cuda.synchronize()
    return HipRun(h, ws, None, None, None, None, 0, buf, None, None)


CASES = [
    # name, T, H, E, k, mode, neg
    ("b1", 40, 256, 8, 4, "mxfp8", 0.1),
    ("b2", 33, 96, 7, 3, "mxfp4", 0.3),
    ("b3", 50, 1024, 16, 8, "fp8_b128", 0.0),
    ("b4", 20, 1056, 5, 6, "int8_token", 0.2),
    ("b5", 64, 128, 32, 16, "none", 0.1),
    ("b6", 9, 7168, 256, 8, "mxfp8", 0.0),
    ("b7", 0, 256, 8, 4, "mxfp8", 0.0),
    ("b8", 30, 512, 16, 8, "fp8_b128_ue8m0", 0.1),
    ("b9", 30, 384, 16, 4, "fp8_b128_pow2", 0.0),
]


@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(ep, case, weighted):
    name, T, H, E, k, mode, neg = case
    print(f"\n[case] backward {name} T={T} H={H} E={E} k={k} {mode} weighted={weighted}", flush=True)
    sys.stdout.flush()
    w = W.Workload(name, T, H, E, k, "int64", mode, "uniform", neg_frac=neg, seed=6000 + T + H)
    inp = W.make_inputs(w)
    grad = W.make_inputs(W.Workload("g", T, H, E, k, "int64", mode, "uniform", seed=7000 + T))["x"]
    run = _run(ep, w, inp, grad, weighted)
    lay = OL.layout(inp["topk_idx"], E, T)
    rb = OB.combine_backward(grad, lay, mode, inp["topk_weights"] if weighted else None)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R])
    assert np.array_equal(scales[:R], rb.scales[:R])


def test_backward_full_size_sampled(ep):
    """The large workload's routing at full size, MXFP8 gradient rows (the
    format the page uses for this path): about 3000 sampled tokens (every
    routed row of each), the oracle's rows quantised in worker processes."""
    print("\n[case] backward full size T=16384 H=7168 mxfp8", flush=True)
    base = W.WORKLOADS["large"]
    w = W.scaled(base, mode="mxfp8")
    inp = W.make_inputs(w)
    grad = W.make_expert_out(w, rows=w.T)
    run = _run(ep, w, inp, grad, True)
    lay = OL.layout(inp["topk_idx"], w.E, w.T)
    toks = sample_tokens(w, inp["topk_idx"], n=2048)
    want = backward_parallel(grad, lay, w.mode, inp["topk_weights"], toks)
    rows = sorted(want)
    data, scales = recv_rows(ep, run, w, rows)
    assert np.array_equal(data, np.stack([want[r][0] for r in rows]))
    assert np.array_equal(scales, np.stack([want[r][1] for r in rows]))


def test_backward_full_size_unweighted(ep):
    """The large workload's routing at full size without weights, MXFP4 rows:
    every routed row (the oracle's unweighted rows are its row quantiser on
    grad[t], run in worker processes for all 16384 tokens)."""
    print("\n[case] backward full size unweighted T=16384 H=7168 mxfp4", flush=True)
    w = W.WORKLOADS["large"]
    inp = W.make_inputs(w)
    grad = W.make_expert_out(w, rows=w.T)
    run = _run(ep, w, inp, grad, False)
    lay = OL.layout(inp["topk_idx"], w.E, w.T)
    want = dispatch_parallel(grad, lay, w.mode)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], want.data[:R])
    assert np.array_equal(scales[:R], want.scales[:R])


@pytest.mark.parametrize("mode", ["mxfp8", "mxfp4"])
def test_backward_every_bf16_pattern(ep, mode):
    """Weighted reverse dispatch of all 65536 bf16 patterns (NaN/Inf replaced
    by 0), shuffled and sorted into rows, plus rows of zeros, subnormals and
    near-overflow values, under weights that include 1, -1, tiny and
    subnormal ones (no product overflows): every product rounded to bf16,
    every block maximum and every clamp at the top of the code range is
    compared with the oracle bit for bit."""
    from oracle import codecs
    print(f"\n[case] backward every bf16 pattern {mode}", flush=True)
    H = 1024
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_bits_to_f32(pats)
    pats[~np.isfinite(f)] = 0
    rng = np.random.default_rng(13)
    extra = np.zeros((4, H), np.uint16)
    extra[1, :] = 0x0001
    extra[2, :] = 0x7F7F
    extra[3, ::2] = 0x8000
    grad = np.concatenate([rng.permutation(pats).reshape(-1, H), np.sort(pats).reshape(-1, H), extra])
    T, k, E = grad.shape[0], 2, 8
    w = W.Workload("bp", T, H, E, k, "int64", mode, "uniform", seed=6100)
    inp = W.make_inputs(w)
    wts = inp["topk_weights"].copy()
    wts[0::7, 0] = 1.0
    wts[1::7, 1] = -1.0
    wts[2::7, 0] = np.float32(2.0 ** -120)
    wts[3::7, 1] = np.float32(0.75)
    wts[4::7, 0] = np.float32(1.5 * 2.0 ** -140)
    inp["topk_weights"] = wts
    run = _run(ep, w, inp, grad, True)
    lay = OL.layout(inp["topk_idx"], E, T)
    rb = OB.combine_backward(grad, lay, mode, wts)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(scales[:R], rb.scales[:R])
    assert np.array_equal(data[:R], rb.data[:R])
