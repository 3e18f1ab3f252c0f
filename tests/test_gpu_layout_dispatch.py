"""GPU parity of ep_layout_dispatch (layout and dispatch in one call) against
the CPU oracle, and against the separate ep_layout_ex + ep_dispatch calls.

Compact layouts and capacity blocks of at most 2048 (token, j) pairs take
the one-launch path, in which every dispatch workgroup counts its own
receive rows from the ids (with capacity blocks also layout workgroups that
mark each block's free rows); aligned blocks and larger inputs take the two
launches of the separate calls.  Every case below is
compared with the oracle bit-exactly (layout, codes, scales, receive
weights, combine), on both sides of the 2048-pair limit, with the edge cases
of the fuzz set (empty input, capacity above T, pairs routed nowhere,
duplicate experts, out-of-range ids, k = 1 and 16, E = 1 and 512, int32 and
int64 ids, the widest int8 rows).
"""

import sys
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from tests.hip_path import DEV, canary_buffer, read_layout, recv_rows, run_layout, run_layout_dispatch, \
    run_path, to_dev
from tests.oracle_path import oracle_run
from tests.test_gpu_fuzz import CASES
from tests.test_gpu_parity import check_combine, check_layout

pytestmark = pytest.mark.gpu

SMALL = ["small", "decode8", "a5fused", "decode"]


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _check(ep, w, inp, y=None):
    run = run_path(ep, w, inp, expert_out=y, fused=True)
    lay, rb, out = oracle_run(w, inp, y)
    check_layout(run, lay)
    rows = lay.valid_rows()          # rows that hold a pair (padding rows are unspecified)
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[rows], rb.data[rows])
    assert np.array_equal(scales[rows], rb.scales[rows])
    assert np.array_equal(run.recv_weights[rows].cpu().numpy(), rb.weights[rows])
    if run.out is not None and w.T:
        check_combine(w, run.out, out)
    return run, lay


@pytest.mark.parametrize("name", SMALL)
def test_workload(ep, name):
    w = W.WORKLOADS[name]
    _announce(f"layout_dispatch {name} T={w.T} H={w.H} E={w.E} k={w.k} {w.mode}")
    inp = W.make_inputs(w)
    y = W.make_expert_out(w) if w.combine_input == "normal" else None
    _check(ep, w, inp, y)


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_fuzz_case(ep, case):
    seed, T, H, E, k, mode, idt, neg, tmax, cin = case
    _announce(f"layout_dispatch fuzz seed={seed} T={T} H={H} E={E} k={k} {mode} {idt} neg={neg} tmax={tmax}")
    w = W.Workload(f"fz{seed}", T, H, E, k, idt, mode, "uniform", neg_frac=neg, combine_input=cin,
                   seed=5000 + seed, num_max_tokens=tmax)
    inp = W.make_inputs(w)
    if seed % 3 == 0 and k > 1 and T:
        inp["topk_idx"] = W.with_duplicates(inp["topk_idx"], seed)
    y = W.make_expert_out(w) if cin == "normal" else None
    _check(ep, w, inp, y)


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_fuzz_case_capacity(ep, case):
    """The fuzz set with capacity blocks of about the average load per expert
    (at least one row), so that many blocks overflow and drop pairs: the one
    launch up to 2048 pairs, the separate calls above."""
    seed, T, H, E, k, mode, idt, neg, tmax, cin = case
    cap = max(1, (T * k) // E)
    _announce(f"layout_dispatch capacity fuzz seed={seed} T={T} H={H} E={E} k={k} {mode} {idt} cap={cap}")
    w = W.Workload(f"fc{seed}", T, H, E, k, idt, mode, "uniform", neg_frac=neg, combine_input=cin,
                   seed=5000 + seed, num_max_tokens=tmax, expert_capacity=cap)
    inp = W.make_inputs(w)
    if seed % 3 == 0 and k > 1 and T:
        inp["topk_idx"] = W.with_duplicates(inp["topk_idx"], seed)
    y = W.make_expert_out(w) if cin == "normal" else None
    _check(ep, w, inp, y)


# both sides of the 2048-pair limit, compact and padded layouts
EDGES = [
    # name, T, H, E, k, mode, idx_dtype, neg_frac, t_max, row_align, capacity
    ("at_limit", 256, 7168, 256, 8, "fp8_b128", "int64", 0.05, 256, 1, 0),
    ("past_limit", 2049, 256, 64, 1, "mxfp8", "int32", 0.0, 2049, 1, 0),
    ("k16_at_limit", 128, 512, 512, 16, "mxfp4", "int32", 0.1, 200, 1, 0),
    ("aligned", 64, 1024, 16, 8, "mxfp8", "int64", 0.1, 64, 128, 0),
    ("capacity", 64, 1024, 16, 8, "int8_token", "int64", 0.1, 64, 1, 24),
    # capacity blocks: the page's [experts, max tokens, hidden] at decode
    # (32768 rows, 8 layout workgroups), overflowing blocks, both sides of
    # the pair limit, one expert
    ("capacity_decode", 128, 7168, 256, 8, "fp8_b128", "int64", 0.1, 128, 1, 128),
    ("capacity_overflow", 200, 512, 8, 8, "mxfp8", "int32", 0.05, 200, 1, 150),
    ("capacity_at_limit", 256, 1024, 64, 8, "mxfp4", "int64", 0.0, 256, 1, 40),
    ("capacity_past_limit", 257, 256, 64, 8, "int8_token", "int64", 0.0, 257, 1, 48),
    ("capacity_one_expert", 100, 256, 1, 1, "none", "int32", 0.2, 100, 1, 64),
]


@pytest.mark.parametrize("case", EDGES, ids=[c[0] for c in EDGES])
def test_limits_and_padded(ep, case):
    name, T, H, E, k, mode, idt, neg, tmax, align, cap = case
    _announce(f"layout_dispatch {name} T={T} H={H} E={E} k={k} {mode} align={align} cap={cap}")
    w = W.Workload(name, T, H, E, k, idt, mode, "uniform", neg_frac=neg, combine_input="identity",
                   seed=6100 + T, num_max_tokens=tmax, row_align=align, expert_capacity=cap)
    _check(ep, w, W.make_inputs(w))


def test_out_of_range_ids_set_status(ep):
    _announce("layout_dispatch out-of-range ids")
    w = W.Workload("oor", 50, 64, 10, 4, "int64", "mxfp8", "uniform", combine_input="identity", seed=77)
    inp = W.make_inputs(w)
    idx = inp["topk_idx"].copy()
    idx[3, 1], idx[7, 0], idx[20, 3], idx[21, 2] = 10, -2, 1 << 40, -(1 << 40)
    inp["topk_idx"] = idx
    run, lay = _check(ep, w, inp)
    assert run.status == 1 and lay.status == 1
    assert run.slot[3, 1] == -1 and run.slot[7, 0] == -1 and run.slot[20, 3] == -1 and run.slot[21, 2] == -1


@pytest.mark.parametrize("T,tmax", [(128, 16384), (0, 4096), (1, 2048)])
def test_capacity_far_above_tokens(ep, T, tmax):
    """A decode-sized batch with a large num_max_dispatch_tokens: the one
    launch leaves up to 131072 rows free, cleared by every span workgroup
    (or, with no token, by the layout workgroup); row_src and the whole
    receive buffer equal those of the separate calls."""
    _announce(f"layout_dispatch T={T} t_max={tmax}")
    w = W.Workload("tmax", T, 7168, 256, 8, "int64", "fp8_b128", "uniform", neg_frac=0.1, seed=83,
                   num_max_tokens=tmax)
    inp = W.make_inputs(w)
    x, wts = to_dev(inp["x"]), to_dev(inp["topk_weights"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    ra, rb = canary_buffer(total), canary_buffer(total)
    ha, wsa, rca = run_layout_dispatch(ep, w, inp["topk_idx"], x, wts, ra, None)
    hb, wsb, rcb = run_layout(ep, w, inp["topk_idx"])
    ep.ep_dispatch(hb, x, w.H, w.mode, rb)
    la, lb = read_layout(ep, ha, wsa, rca, w), read_layout(ep, hb, wsb, rcb, w)
    for key in ("recv_count", "offsets", "slot", "row_src"):
        assert np.array_equal(la[key], lb[key]), key
    assert np.all(la["row_src"][T * w.k:] == -1)
    assert la["status"] == lb["status"]
    assert torch.equal(ra, rb)


def test_same_bytes_as_separate_calls(ep):
    """Whole receive buffer (canaries of unused rows included), receive
    weights, layout arrays and running statistics equal those of
    ep_layout_ex + ep_dispatch, over three calls in a row."""
    _announce("layout_dispatch vs separate calls")
    w = W.Workload("sep", 100, 2048, 40, 6, "int32", "mxfp4", "uniform", neg_frac=0.1, seed=81,
                   num_max_tokens=130)
    inp = W.make_inputs(w)
    inp["topk_idx"] = W.with_duplicates(inp["topk_idx"], 3)
    x, wts = to_dev(inp["x"]), to_dev(inp["topk_weights"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    cum_a = torch.full((w.E,), 3, dtype=torch.int32, device=DEV)
    cum_b = cum_a.clone()
    for it in range(3):
        ra, rb = canary_buffer(total), canary_buffer(total)
        wa = torch.full((w.max_rows,), float("nan"), device=DEV)
        wb = wa.clone()
        ha, wsa, rca = run_layout_dispatch(ep, w, inp["topk_idx"], x, wts, ra, wa, cum_a)
        hb, wsb, rcb = run_layout(ep, w, inp["topk_idx"], cum_b)
        ep.ep_dispatch(hb, x, w.H, w.mode, rb, wts, wb)
        la, lb = read_layout(ep, ha, wsa, rca, w), read_layout(ep, hb, wsb, rcb, w)
        for key in ("recv_count", "offsets", "slot", "row_src"):
            assert np.array_equal(la[key], lb[key]), key
        assert la["status"] == lb["status"]
        assert torch.equal(ra, rb)
        assert np.array_equal(wa.cpu().numpy(), wb.cpu().numpy(), equal_nan=True)
        assert torch.equal(cum_a, cum_b)


@pytest.mark.parametrize("T,E,k,cap,mode,idt", [
    (100, 40, 6, 20, "mxfp4", "int32"),       # overflowing blocks, duplicate experts, out-of-range ids
    (128, 256, 8, 128, "fp8_b128", "int64"),  # decode shape, 8 layout workgroups
    (0, 16, 4, 32, "mxfp8", "int64"),         # no token: the layout workgroups mark every row free
], ids=["overflow", "decode", "empty"])
def test_capacity_same_bytes_as_separate_calls(ep, T, E, k, cap, mode, idt):
    """Capacity blocks through the one launch: whole receive buffer (canaries
    of unused rows included), receive weights, layout arrays, status and
    running statistics equal those of ep_layout_ex + ep_dispatch, over three
    calls in a row."""
    _announce(f"layout_dispatch capacity vs separate calls T={T} E={E} k={k} cap={cap} {mode} {idt}")
    w = W.Workload("capsep", T, 1024, E, k, idt, mode, "uniform", neg_frac=0.1, combine_input="identity",
                   seed=91 + T, num_max_tokens=max(T, 1), expert_capacity=cap)
    inp = W.make_inputs(w)
    if T and k > 1:
        inp["topk_idx"] = W.with_duplicates(inp["topk_idx"], 5)
    if T >= 30:
        idx = inp["topk_idx"].copy()
        idx[3, 0], idx[17, k - 1] = E, -5               # out of range: status bit, pair dropped
        inp["topk_idx"] = idx
    x, wts = to_dev(inp["x"]), to_dev(inp["topk_weights"])
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode)
    cum_a = torch.full((w.E,), 3, dtype=torch.int32, device=DEV)
    cum_b = cum_a.clone()
    for it in range(3):
        ra, rb = canary_buffer(total), canary_buffer(total)
        wa = torch.full((w.max_rows,), float("nan"), device=DEV)
        wb = wa.clone()
        ha, wsa, rca = run_layout_dispatch(ep, w, inp["topk_idx"], x, wts, ra, wa, cum_a)
        hb, wsb, rcb = run_layout(ep, w, inp["topk_idx"], cum_b)
        ep.ep_dispatch(hb, x, w.H, w.mode, rb, wts, wb)
        la, lb = read_layout(ep, ha, wsa, rca, w), read_layout(ep, hb, wsb, rcb, w)
        for key in ("recv_count", "offsets", "slot", "row_src"):
            assert np.array_equal(la[key], lb[key]), key
        assert la["status"] == lb["status"]
        assert torch.equal(ra, rb)
        assert np.array_equal(wa.cpu().numpy(), wb.cpu().numpy(), equal_nan=True)
        assert torch.equal(cum_a, cum_b)
    lay, _, _ = oracle_run(w, inp)
    check_layout(SimpleNamespace(recv_count=la["recv_count"], offsets=la["offsets"], slot=la["slot"],
                                 row_src=la["row_src"], status=la["status"]), lay)
