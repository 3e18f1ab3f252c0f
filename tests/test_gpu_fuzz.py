"""GPU edge cases and randomized shapes, each against the oracle.

Covers: empty input (T = 0), capacity larger than T, tokens with no routed
pair, duplicate experts in a row, out-of-range ids (status bit), k = 1 and
k = 16, E = 1 and E = 512, hidden sizes that are and are not multiples of 128
(MX scale packing), ragged tails of the row tiling, int32 and int64 ids, the
multi-workgroup layout path (more than 6144 pairs) and both sides of that limit, every bf16 bit pattern
through every quantiser, blocks of zeros, subnormals and huge values (for the
power-of-two per-128 scales this includes the last kept exponent, -127, and
the zeroed blocks below it).
"""

import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import codecs
from tests.hip_path import run_path, recv_rows, run_layout, read_layout, to_dev, DEV
from tests.oracle_path import oracle_run
from tests.test_gpu_parity import check_combine, check_layout

pytestmark = pytest.mark.gpu

MODES = ["none", "int8_token", "fp8_b128", "mxfp8", "mxfp4", "fp8_b128_pow2", "fp8_b128_ue8m0"]


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _full_check(ep, w, inp, y=None):
    run = run_path(ep, w, inp, expert_out=y)
    lay, rb, out = oracle_run(w, inp, y)
    check_layout(run, lay)
    R = lay.num_rows
    data, scales = recv_rows(ep, run, w)
    assert np.array_equal(data[:R], rb.data[:R])
    assert np.array_equal(scales[:R], rb.scales[:R])
    assert np.array_equal(run.recv_weights[:R].cpu().numpy(), rb.weights[:R])
    if run.out is not None and w.T:
        check_combine(w, run.out, out)
    return run, lay


CASES = [
    # seed, T, H, E, k, mode, idx_dtype, neg_frac, t_max, combine_input
    (1, 0, 256, 8, 4, "mxfp8", "int64", 0.0, 16, "identity"),
    (2, 5, 32, 1, 1, "none", "int32", 0.0, 5, "normal"),
    (3, 33, 96, 7, 3, "mxfp4", "int64", 0.3, 40, "identity"),
    (4, 17, 160, 512, 16, "mxfp8", "int32", 0.1, 17, "identity"),
    (5, 64, 384, 300, 16, "fp8_b128", "int64", 0.5, 100, "normal"),
    (6, 40, 1056, 5, 8, "int8_token", "int64", 0.0, 40, "identity"),
    (7, 9, 7168, 256, 8, "mxfp4", "int64", 1.0, 9, "normal"),          # every pair -1
    (8, 100, 2080, 64, 6, "none", "int32", 0.2, 128, "normal"),
    (9, 3000, 128, 33, 7, "mxfp8", "int64", 0.05, 3000, "identity"),    # multi-block layout
    (10, 2500, 64, 512, 16, "int8_token", "int32", 0.0, 2600, "identity"),
    (11, 12, 16384, 16, 4, "int8_token", "int64", 0.0, 12, "identity"),  # largest int8 tile
    (12, 6, 8192, 4, 2, "mxfp4", "int32", 0.0, 6000, "normal"),           # capacity >> T
    (13, 50, 640, 16, 4, "fp8_b128_pow2", "int64", 0.1, 60, "identity"),
    (14, 3000, 512, 64, 8, "fp8_b128_ue8m0", "int32", 0.05, 3000, "identity"),  # multi-block layout
    (15, 7, 384, 8, 2, "fp8_b128_ue8m0", "int64", 0.0, 7, "identity"),     # 3 scale bytes per row
    (16, 128, 7168, 256, 8, "fp8_b128_pow2", "int64", 0.1, 128, "identity"),
    (17, 768, 256, 48, 8, "mxfp8", "int64", 0.1, 768, "identity"),     # one-workgroup layout at 6144 pairs
    (18, 769, 256, 48, 8, "none", "int32", 0.0, 769, "normal"),         # 6152 pairs: two launches
    (19, 256, 512, 64, 8, "mxfp4", "int64", 0.05, 300, "identity"),     # spare receive rows past R
    (20, 2049, 128, 32, 1, "int8_token", "int32", 0.0, 2049, "identity"),  # k = 1, smallest int8 row
    (21, 3, 65536, 4, 2, "int8_token", "int64", 0.0, 3, "identity"),    # largest hidden: 1024 threads x 8 vectors
    (22, 5, 65504, 6, 3, "mxfp4", "int32", 0.0, 5, "normal"),           # largest hidden that is not a multiple of 128
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_fuzz_case(ep, case):
    seed, T, H, E, k, mode, idt, neg, tmax, cin = case
    _announce(f"fuzz seed={seed} T={T} H={H} E={E} k={k} {mode} {idt} neg={neg} tmax={tmax} {cin}")
    w = W.Workload(f"fz{seed}", T, H, E, k, idt, mode, "uniform", neg_frac=neg, combine_input=cin,
                   seed=5000 + seed, num_max_tokens=tmax)
    inp = W.make_inputs(w)
    if seed % 3 == 0 and k > 1 and T:
        inp["topk_idx"] = W.with_duplicates(inp["topk_idx"], seed)
    y = W.make_expert_out(w) if cin == "normal" else None
    _full_check(ep, w, inp, y)


def test_out_of_range_ids_set_status(ep):
    w = W.Workload("oor", 50, 64, 10, 4, "int64", "mxfp8", "uniform", combine_input="identity", seed=77)
    _announce("out-of-range ids")
    inp = W.make_inputs(w)
    idx = inp["topk_idx"].copy()
    idx[3, 1], idx[7, 0], idx[20, 3] = 10, -2, 1 << 40
    inp["topk_idx"] = idx
    run, lay = _full_check(ep, w, inp)
    assert run.status == 1 and lay.status == 1
    assert run.slot[3, 1] == -1 and run.slot[7, 0] == -1 and run.slot[20, 3] == -1


@pytest.mark.parametrize("mode", MODES)
def test_every_bf16_pattern(ep, mode):
    """All 65536 bf16 patterns (NaN/Inf replaced by 0) through each quantiser,
    shuffled so that blocks mix magnitudes, plus blocks of zeros, subnormals
    and near-overflow values."""
    _announce(f"every bf16 pattern through {mode}")
    H = 1024
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_bits_to_f32(pats)
    pats[~np.isfinite(f)] = 0
    rng = np.random.default_rng(11)
    shuffled = rng.permutation(pats)
    sorted_ = np.sort(pats)                      # blocks of similar magnitude
    extra = np.zeros((8, H), np.uint16)
    extra[1, :] = 0x0001                          # smallest subnormal everywhere
    extra[2, :] = rng.integers(0, 0x80, H).astype(np.uint16) | np.uint16(0x8000) * rng.integers(0, 2, H).astype(np.uint16)
    extra[3, :] = 0x7F7F                          # largest finite
    extra[4, ::2] = 0x8000                        # negative zeros
    extra[5, :] = (0x3F80 + rng.integers(0, 128, H)).astype(np.uint16)
    x = np.concatenate([shuffled.reshape(-1, H), sorted_.reshape(-1, H), extra])
    T = x.shape[0]
    w = W.Workload("pat", T, H, 4, 2, "int64", mode, "uniform", combine_input="identity", seed=91)
    inp = W.make_inputs(w)
    inp["x"] = x
    _full_check(ep, w, inp)


def test_multiblock_layout_large(ep):
    """More than 16384 pairs with a skewed expert mix, int32 ids, duplicates,
    compared with the oracle on every output of the layout."""
    _announce("multi-block layout 40000x8")
    w = W.Workload("mb", 40000, 32, 512, 8, "int32", "none", "zipf", neg_frac=0.02, seed=123,
                   num_max_tokens=41000)
    inp = W.make_inputs(w)
    idx = W.with_duplicates(inp["topk_idx"], 5)
    from oracle import layout as L
    cum = torch.arange(w.E, dtype=torch.int32, device=DEV)
    h, ws, rc = run_layout(ep, w, idx, cum)
    got = read_layout(ep, h, ws, rc, w)
    cum_ref = np.arange(w.E, dtype=np.int32)
    lay = L.layout(idx, w.E, w.t_max, cum_stats=cum_ref)
    assert np.array_equal(got["recv_count"], lay.count)
    assert np.array_equal(got["offsets"], lay.offsets.astype(np.int32))
    assert np.array_equal(got["slot"], lay.slot)
    assert np.array_equal(got["row_src"], lay.row_src)
    assert got["status"] == 0
    assert np.array_equal(cum.cpu().numpy(), cum_ref)


def test_single_block_layout_cum_stats(ep):
    _announce("single-block layout cumulative stats")
    w = W.Workload("cs", 100, 32, 20, 3, "int64", "none", "uniform", neg_frac=0.1, seed=55)
    inp = W.make_inputs(w)
    from oracle import layout as L
    cum = torch.full((w.E,), 5, dtype=torch.int32, device=DEV)
    cum_ref = np.full(w.E, 5, np.int32)
    for _ in range(3):                               # accumulates across calls
        h, ws, rc = run_layout(ep, w, inp["topk_idx"], cum)
        L.layout(inp["topk_idx"], w.E, w.t_max, cum_stats=cum_ref)
    torch.cuda.synchronize()
    assert np.array_equal(cum.cpu().numpy(), cum_ref)


def test_low_latency_wrappers(ep):
    """The page-shaped Python wrappers return the page's shapes and the same
    bytes as the oracle."""
    _announce("low_latency_dispatch / low_latency_combine wrappers")
    w = W.Workload("ll", 24, 256, 8, 4, "int64", "mxfp4", "uniform", neg_frac=0.1, seed=31,
                   combine_input="identity")
    inp = W.make_inputs(w)
    x = to_dev(inp["x"])
    idx = to_dev(inp["topk_idx"])
    wts = to_dev(inp["topk_weights"])
    (data, scales), recv_count, handle, ev, hook = ep.low_latency_dispatch(
        x, idx, w.T, w.E, use_fp8=True, use_mxfp4=True, topk_weights=wts)
    assert data.shape == (w.max_rows, w.H // 2) and data.dtype == torch.float4_e2m1fn_x2
    assert scales.shape == (w.max_rows * w.H // 32,) and scales.dtype == torch.float8_e8m0fnu
    lay, rb, _ = oracle_run(w, inp)
    R = lay.num_rows
    assert np.array_equal(recv_count.cpu().numpy(), lay.count)
    assert np.array_equal(data.view(torch.uint8).cpu().numpy()[:R], rb.data[:R])
    assert np.array_equal(scales.view(torch.uint8).cpu().numpy()[: R * w.H // 32], rb.scales[:R].reshape(-1))
    # combine of bf16 expert outputs through the wrapper
    y = W.make_expert_out(w)
    out, _, _ = ep.low_latency_combine(to_dev(y), idx, wts, handle)
    w2 = W.Workload("ll", 24, 256, 8, 4, "int64", "none", "uniform", neg_frac=0.1, seed=31,
                    combine_input="normal")
    _, _, want = oracle_run(w2, inp, y)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
