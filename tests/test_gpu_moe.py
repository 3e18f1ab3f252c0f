"""GPU parity of the expert MLP (ep_moe_gmm1 / ep_moe_gmm2) against the
float64 oracle, on the same seeded inputs.

The matrix cores sum each 64-product step with less than float32 precision,
so the bars are bounds, not bit equality.  Every bound is derived in
``tests/moe_bounds.py`` from one stated model of the matrix-core step
(at least 11 fraction bits below the step's largest product; checked on the
device by ``tests/test_gpu_mfma_model.py``) and from the oracle's own
values; every comparison is against the oracle's chain:

* GMM1 with bf16 output: each element within B1 (the model through
  silu(g) u) plus its bf16 rounding of the oracle's exact a;
* GMM1 with MXFP8 output: scale bytes among the exponents the block maximum
  can reach within B1 (nearly always only the oracle's), every code between
  the codes of a - B1 and a + B1 -- so equal to the oracle's code wherever a
  is not within B1 of an e4m3 rounding boundary; no share of differing codes
  is allowed beyond that;
* GMM2 rows against the oracle's exact W2 deq(q): the codes that may differ
  move a row by at most sum |W2| D, plus the model's bound and the bf16
  rounding;
* the whole path (dispatch, GMM1, requant, GMM2, combine) against the
  oracle's output: each element within the expert rows' bounds carried
  through |w|, float32 accumulation and the final bf16 rounding; and, on the
  full-size share workloads, every routed row within the 2e-2 relative L2
  error stated for a quantised combine.

Rows holding no pair are never written (their canaries survive).
"""

import sys

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import codecs, dispatch as OD, moe as OM
from tests.hip_path import DEV, canary_buffer, to_dev, NAN_BF16
from tests import moe_bounds as MB
from tests.moe_path import gpu_moe, oracle_moe, read_slots

pytestmark = pytest.mark.gpu

ROW_REL = 2e-2          # per-row relative L2 error of a quantised combine


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _bf16_rows(buf, rows, width):
    return buf[: rows * width * 2].view(torch.int16).view(rows, width).cpu().numpy().view(np.uint16)


def _f64(bits):
    return codecs.bf16_bits_to_f32(bits).astype(np.float64)


def _check_gmm1_bf16(got_bits, xv, w1v, want_a):
    a, B1 = MB.gmm1_bound(xv, w1v)
    assert np.allclose(a, want_a, rtol=1e-12, atol=1e-300)       # the same exact a as the oracle's
    bound = B1 + MB._ulp_bf16(np.abs(a) + B1) / 2.0
    got = _f64(got_bits)
    assert np.all(np.isfinite(got))
    err = np.abs(got - a)
    assert np.all(err <= bound), f"worst err/bound {np.max(err / bound):.3g}"
    return float(np.max(err / bound))


def _expert_mats(inp, e, rb, rows):
    xv = OM.mx_dequant(rb.data[rows], rb.scales[rows])
    return xv, OM.mx_dequant(inp["w1_codes"][e], inp["w1_scales"][e]), \
        OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e])


def check_chain(ep, w, inp, res, lay, rb, per, out, tokens=None, gmm2=True, row_rel=None):
    """The GPU's requant, GMM2 rows and combine output against the oracle's
    chain with the derived bounds; returns a summary dict."""
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    y_gpu = _bf16_rows(res["y"], lay.max_rows, w.H) if gmm2 else None
    row_bound = np.zeros((lay.max_rows, w.H))
    y_exact = np.zeros((lay.max_rows, w.H))
    st = {"codes": 0, "ambiguous": 0, "differ": 0, "scale_ranges": 0, "blocks": 0, "gmm2_worst": 0.0}
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        xv, w1v, w2v = _expert_mats(inp, e, rb, rows)
        _, B1 = MB.gmm1_bound(xv, w1v)
        a32 = ent["a"].astype(np.float32)
        D, s = MB.check_requant(a.data[rows], a.scales[rows], a32, B1, ent["q"], ent["qs"])
        for key in s:
            st[key] += s[key]
        if not gmm2:
            continue
        want_v = OM.mx_dequant(ent["q"], ent["qs"])
        bound, _ = MB.gmm2_bound(want_v, D, w2v, ent["y"])
        err = np.abs(_f64(y_gpu[rows]) - ent["y"])
        assert np.all(err <= bound), f"expert {e}: GMM2 rows outside their bounds, worst {np.max(err / bound):.3g}"
        st["gmm2_worst"] = max(st["gmm2_worst"], float(np.max(err / bound)))
        row_bound[rows], y_exact[rows] = bound, ent["y"]
    if gmm2 and out is not None:
        toks = np.arange(w.T) if tokens is None else np.asarray(tokens)
        got = _f64(res["out"][toks])
        want = _f64(out)
        cb = MB.combine_bound(row_bound, y_exact, lay.slot[toks], inp["topk_weights"][toks], want)
        err = np.abs(got - want)
        assert np.all(err <= cb), f"combine outside its bound, worst {np.max(err / cb):.3g}"
        st["combine_worst"] = float(np.max(err / cb))
        routed = np.linalg.norm(want, axis=1) > 0
        rel = np.linalg.norm(got - want, axis=1) / np.maximum(np.linalg.norm(want, axis=1), 1e-300)
        st["row_rel_worst"] = float(np.max(rel[routed])) if routed.any() else 0.0
        assert np.all(got[~routed] == 0)
        if row_rel is not None:
            assert st["row_rel_worst"] <= row_rel, f"worst row relative error {st['row_rel_worst']:.3g}"
    print("chain: " + ", ".join(f"{k} {v:.3g}" if isinstance(v, float) else f"{k} {v}" for k, v in st.items()))
    return st


@pytest.mark.parametrize("pass_count", [True, False])
def test_gmm1_bf16_small(ep, pass_count):
    w = W.MOE_WORKLOADS["moe_small"]
    _announce(f"gmm1 bf16 moe_small pass_count={pass_count}")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="none", pass_count=pass_count, stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="bf16")
    got = _bf16_rows(res["a"], lay.max_rows, w.I)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        xv, w1v, _ = _expert_mats(inp, e, rb, rows)
        _check_gmm1_bf16(got[rows], xv, w1v, ent["a"])
    free = np.nonzero(lay.row_src < 0)[0]
    assert np.all(got[free] == NAN_BF16)                             # never written


def test_gmm1_mxfp8_small(ep):
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("gmm1 mxfp8 moe_small")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="mxfp8", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="mxfp8")
    check_chain(ep, w, inp, res, lay, rb, per, None, gmm2=False)


@pytest.mark.parametrize("out_quant", ["none", "mxfp8"])
def test_gmm1_silu_extremes(ep, out_quant):
    """The gate rows' scale bytes raised by 5 (x32): |g| reaches the
    hundreds, so in float32 e^-g overflows (silu -> -0; the exact value is
    below 1e-36), underflows (silu -> g), and near g = -88 its reciprocal
    1 / (1 + e^-g) is subnormal.  Every element stays within the derived
    bound of the oracle's exact a."""
    w = W.MOE_WORKLOADS["moe_small"]
    _announce(f"gmm1 silu extremes moe_small {out_quant}")
    inp = dict(W.make_moe_inputs(w))
    s = inp["w1_scales"].copy()
    s[:, : w.I] = np.minimum(s[:, : w.I].astype(np.int32) + 5, 254).astype(np.uint8)
    inp["w1_scales"] = s
    res = gpu_moe(ep, w, inp, out_quant=out_quant, stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="bf16" if out_quant == "none" else "mxfp8")
    g_all = []
    for e, (rows, ent) in enumerate(per):
        if ent is not None:
            xv, w1v, _ = _expert_mats(inp, e, rb, rows)
            g_all.append((xv @ w1v[: w.I].T).ravel())
    g_all = np.concatenate(g_all)
    # the regimes are reached: overflow of e^-g, its underflow, and the
    # subnormal reciprocal window
    assert (g_all < -88.8).sum() > 100 and (g_all > 88.8).sum() > 100
    assert ((g_all > -88.7) & (g_all < -87.4)).sum() > 10
    if out_quant == "none":
        got = _bf16_rows(res["a"], lay.max_rows, w.I)
        for e, (rows, ent) in enumerate(per):
            if ent is not None:
                xv, w1v, _ = _expert_mats(inp, e, rb, rows)
                _check_gmm1_bf16(got[rows], xv, w1v, ent["a"])
    else:
        check_chain(ep, w, inp, res, lay, rb, per, None, gmm2=False)


def test_gmm2_on_shared_input(ep):
    """GMM2 alone: both sides read the same synthetic MXFP8 activations."""
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("gmm2 on synthetic MXFP8 rows, moe_small")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="mxfp8", stop_after="gmm1")
    h = res["handle"]
    rows = h.max_rows
    ac, asc = W.make_mx_weights(w.seed + 9, 1, rows, w.I)
    shared = OD.RecvBuffer("mxfp8", w.I, rows, ac[0], asc[0], None)
    a_buf = to_dev(shared.to_bytes())
    y = canary_buffer(rows * w.H * 2)
    ep.ep_moe_gmm2(h, a_buf, w.I, w.H, res["w2"][0], res["w2"][1], y, recv_count=res["rc"])
    torch.cuda.synchronize()
    got = _f64(_bf16_rows(y, rows, w.H))
    rc = res["rc"].cpu().numpy()
    _, offs = read_slots(ep, res, w)
    for e in range(w.E_local):
        r = np.arange(offs[e], offs[e] + rc[e])
        if r.size == 0:
            continue
        _, yv = OM.gmm2_rows(ac[0][r], asc[0][r], inp["w2_codes"][e], inp["w2_scales"][e])
        bound, _ = MB.gmm2_bound(OM.mx_dequant(ac[0][r], asc[0][r]), np.zeros((r.size, w.I)),
                                 OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e]), yv)
        err = np.abs(got[r] - yv)
        assert np.all(err <= bound), f"expert {e}: worst err/bound {np.max(err / bound):.3g}"


def test_end_to_end_small(ep):
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("moe end to end, moe_small")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    check_chain(ep, w, inp, res, lay, rb, per, out)


def test_hot_expert_many_chunks_and_empty_experts(ep):
    """One expert with more than 256 rows (several work items), experts with
    none, the aligned layout (padding rows between blocks), bf16 GMM1."""
    w = W.MoeWorkload("moe_hot", 400, 256, 128, 8, 4, 2, seed=1023)
    _announce("moe hot expert / empty experts / aligned blocks")
    inp = W.make_moe_inputs(w)
    idx = inp["topk_idx"].copy()
    idx[:, 0] = 0                                                  # expert 0: 400+ rows
    idx[idx == 2] = -1                                             # expert 2: none
    inp["topk_idx"] = idx
    for row_align in (1, 64):
        res = gpu_moe(ep, w, inp, out_quant="none", row_align=row_align, stop_after="gmm1")
        lay, rb, per, _ = oracle_moe(w, inp, out_mode="bf16", row_align=row_align)
        assert lay.count[0] > 256 and lay.count[2] == 0
        got = _bf16_rows(res["a"], lay.max_rows, w.I)
        for e, (rows, ent) in enumerate(per):
            if ent is None:
                continue
            xv, w1v, _ = _expert_mats(inp, e, rb, rows)
            _check_gmm1_bf16(got[rows], xv, w1v, ent["a"])
        free = np.nonzero(lay.row_src < 0)[0]
        assert np.all(got[free] == NAN_BF16)
    # the whole chain on the aligned blocks
    res = gpu_moe(ep, w, inp, row_align=64)
    lay, rb, per, out = oracle_moe(w, inp, row_align=64)
    check_chain(ep, w, inp, res, lay, rb, per, out)


def test_mixed_tile_widths(ep):
    """A launch with both tile widths (on a 256-CU device): GMM1 of I = 3072
    has 96 four-group or 64 six-group tiles per chunk; with three chunks the
    six-group plan fits one round and the chunk with the most fragments moves
    to four-group tiles.  Expert 0 has 200 rows, a full 160-row chunk (five
    fragments: narrow) and a 40-row one (two fragments: wide); expert 1 has
    60 rows (wide).  bf16 GMM1, then the whole chain, against the oracle."""
    w = W.MoeWorkload("moe_mixed", 260, 256, 3072, 2, 2, 1, seed=1026)
    _announce("moe mixed tile widths: 200 + 60 rows, I=3072")
    inp = W.make_moe_inputs(w)
    idx = np.zeros((w.T, 1), dtype=inp["topk_idx"].dtype)
    idx[200:] = 1
    inp["topk_idx"] = idx
    res = gpu_moe(ep, w, inp, out_quant="none", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="bf16")
    assert list(lay.count) == [200, 60]
    got = _bf16_rows(res["a"], lay.max_rows, w.I)
    for e, (rows, ent) in enumerate(per):
        xv, w1v, _ = _expert_mats(inp, e, rb, rows)
        _check_gmm1_bf16(got[rows], xv, w1v, ent["a"])
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    check_chain(ep, w, inp, res, lay, rb, per, out)


def test_capacity_padded_blocks(ep):
    """The [E, C, ...] receive shape of the low-latency API: every expert
    block has C rows, the hot expert's pairs past the C-th are dropped (slot
    -1, never multiplied), the rest of each block is never written; the
    whole path through combine against the oracle."""
    w = W.MoeWorkload("moe_cap", 200, 256, 128, 8, 4, 2, seed=1026)
    _announce("moe capacity-padded blocks, C = 96")
    inp = W.make_moe_inputs(w)
    idx = inp["topk_idx"].copy()
    idx[:, 0] = 0                                                  # expert 0 wants 200 rows, keeps 96
    inp["topk_idx"] = idx
    cap = 96
    res = gpu_moe(ep, w, inp, expert_capacity=cap)
    lay, rb, per, out = oracle_moe(w, inp, expert_capacity=cap)
    assert lay.max_rows == w.E_local * cap and lay.count[0] == cap and lay.status & 2
    slot, offs = read_slots(ep, res, w)
    assert np.array_equal(slot, lay.slot) and np.array_equal(offs, lay.offsets.astype(np.int32))
    y = _bf16_rows(res["y"], lay.max_rows, w.H)
    free = np.nonzero(lay.row_src < 0)[0]
    assert free.size > 0 and np.all(y[free] == NAN_BF16)          # padding rows never written
    check_chain(ep, w, inp, res, lay, rb, per, out)


@pytest.mark.parametrize("name", ["moe_share", "moe_share32"])
def test_share_full_size(ep, name):
    """The share at full size (hidden 7168, intermediate 3072, 6 local
    experts; 1024 tokens, and 256 whose 1- and 2-fragment chunks put the
    plan on mixed tile widths), every token through the whole path: every
    requantised row, GMM2 row and combine output within its derived bound,
    and every routed token within the 2e-2 relative error of a quantised
    combine."""
    w = W.MOE_WORKLOADS[name]
    _announce(f"{name} full size, every token")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp, parallel=True)
    check_chain(ep, w, inp, res, lay, rb, per, out, row_rel=ROW_REL)


MANY = [
    # 80 experts, H 512, I 256: 320 four-group units against 240 six-group
    # ones, so on a 256-CU device both GEMMs take six-group tiles, the last
    # one partial (16 weight groups = 6 + 6 + 4)
    W.MoeWorkload("moe_wide", 480, 512, 256, 80, 80, 4, seed=1024),
    # 192 experts, H = I = 256: four-group tiles, three units per workgroup
    W.MoeWorkload("moe_rounds", 768, 256, 256, 192, 192, 4, seed=1025),
]


@pytest.mark.parametrize("w", MANY, ids=[m.name for m in MANY])
def test_many_small_experts(ep, w):
    """Many small experts: more work units than CUs (tile width chosen per
    launch, partial last tiles, workgroups walking several units)."""
    _announce(f"{w.name}: {w.E_local} experts, H={w.H}, I={w.I}")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    check_chain(ep, w, inp, res, lay, rb, per, out)


def test_wide_tiles_bf16_output(ep):
    """GMM1 with bf16 output in a launch that takes six-group tiles (the
    partial last tile included), against the per-element bound."""
    w = MANY[0]
    _announce(f"{w.name}: GMM1 bf16 output")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="none", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="bf16")
    got = _bf16_rows(res["a"], lay.max_rows, w.I)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        xv, w1v, _ = _expert_mats(inp, e, rb, rows)
        _check_gmm1_bf16(got[rows], xv, w1v, ent["a"])
    free = np.nonzero(lay.row_src < 0)[0]
    assert np.all(got[free] == NAN_BF16)


def test_recv_count_is_clamped_to_the_block(ep):
    """recv_count entries above the block size (or negative) do not reach
    past the expert's block: the GEMMs then run exactly as with the block
    sizes (recv_count = NULL)."""
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("recv_count clamped to the block")
    inp = W.make_moe_inputs(w)
    ref = gpu_moe(ep, w, inp, out_quant="none", pass_count=False, stop_after="gmm1")
    h = ref["handle"]
    bad = torch.tensor([1 << 40, -5, 1 << 20, 7][: w.E_local], dtype=torch.int64, device=DEV)
    rows_kept = np.minimum(np.maximum(bad.cpu().numpy(), 0), np.diff(read_slots(ep, ref, w)[1]))
    ab, _ = ep.ep_buffer_bytes(h.max_rows, w.I, "none")
    a = canary_buffer(ab)
    ep.ep_moe_gmm1(h, ref["recv"], w.H, w.I, *_packed_w1(ep, inp), "none", a, recv_count=bad)
    torch.cuda.synchronize()
    got = _bf16_rows(a, h.max_rows, w.I)
    want = _bf16_rows(ref["a"], h.max_rows, w.I)
    offs = read_slots(ep, ref, w)[1]
    for e in range(w.E_local):
        r0, n = int(offs[e]), int(rows_kept[e])
        assert np.array_equal(got[r0:r0 + n], want[r0:r0 + n])
        assert np.all(got[r0 + n:offs[e + 1]] == NAN_BF16)            # rows past the clamped count untouched


FUZZ = [
    # T, H, I, E_total, E_local, k, seed: chunks of every fragment count,
    # several chunks per expert, launches with one width or both
    (300, 256, 3072, 4, 3, 2, 1101),
    (500, 384, 1536, 8, 3, 4, 1102),
    (200, 128, 768, 16, 16, 3, 1103),
    (64, 512, 256, 8, 8, 1, 1104),
    (1000, 128, 384, 2, 2, 1, 1105),
    (96, 640, 640, 5, 5, 5, 1106),
    # I = 3072: six-group tiles in one round; three 5-fragment chunks moved
    # to four-group tiles (mixed), and seven chunks with no room to move any
    (768, 256, 3072, 6, 6, 1, 1107),
    (900, 128, 3072, 7, 7, 1, 1109),
    # one expert whose 161 rows make a full chunk and a one-row chunk, and
    # I = 128 (eight GMM1 groups: a full tile and a partial one)
    (161, 256, 256, 1, 1, 1, 1112),
    (130, 128, 128, 3, 3, 2, 1111),
]


@pytest.mark.parametrize("case", FUZZ, ids=[f"f{c[-1]}" for c in FUZZ])
def test_gemm_shapes(ep, case):
    """Assorted shapes through the whole path against the oracle's chain
    (requant, GMM2 rows, combine); rows holding no pair never written."""
    T, H, I, Et, El, k, seed = case
    w = W.MoeWorkload(f"fz{seed}", T, H, I, Et, El, k, seed=seed)
    _announce(f"gemm shapes T={T} H={H} I={I} experts {El}/{Et} k={k}")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    check_chain(ep, w, inp, res, lay, rb, per, out)
    y = _bf16_rows(res["y"], lay.max_rows, w.H)
    free = np.nonzero(lay.row_src < 0)[0]
    assert np.all(y[free] == NAN_BF16)


@pytest.mark.parametrize("inter", [64, 192])
def test_gmm1_inter_not_multiple_of_128(ep, inter):
    """GMM1 takes an intermediate size that is a multiple of 64 (GMM2, which
    reduces over it, needs 128): 64 is one four-group tile, 192 a six-group
    tile and a four-group one; the requant against the oracle's chain, and
    161 + 159 rows (a one-row chunk)."""
    w = W.MoeWorkload(f"i{inter}", 320, 256, inter, 2, 2, 1, seed=1113)
    _announce(f"gmm1 I={inter}")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="mxfp8", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="mxfp8")
    check_chain(ep, w, inp, res, lay, rb, per, None, gmm2=False)


def test_no_routed_rows(ep):
    """Every id -1: no expert has a row, both GEMMs launch with no work unit
    and write nothing, and combine gives +0 rows."""
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("moe with no routed rows")
    inp = W.make_moe_inputs(w)
    inp["topk_idx"] = np.full_like(inp["topk_idx"], -1)
    res = gpu_moe(ep, w, inp)
    h = res["handle"]
    assert int(res["rc"].sum().item()) == 0
    assert torch.all(res["a"].view(torch.int16) == NAN_BF16)
    assert torch.all(res["y"].view(torch.int16) == NAN_BF16)
    assert np.all(res["out"] == 0)
    assert h.max_rows == w.T * w.k


def _packed_w1(ep, inp):
    return ep.pack_moe_weights(to_dev(inp["w1_codes"]), to_dev(inp["w1_scales"]), True)


def _pack_reference(codes, scales, gate_up):
    """The packed layout of ep_moe_pack_weights built with numpy indexing
    from its description in include/ep.h (a permutation of the bytes)."""
    E, N, K = codes.shape
    ks, G, inter = K // 64, N // 32, N // 2
    spans = (ks + 3) // 4
    lanes = np.arange(64)
    r, g = lanes % 32, lanes // 32
    pc = np.zeros((E, G, ks, 2, 64, 16), np.uint8)
    ps = np.zeros((E, G, spans, 64, 4), np.uint8)
    for j in range(G):
        rows = np.where(r < 16, 16 * j + r, inter + 16 * j + r - 16) if gate_up else 32 * j + r
        for s in range(ks):
            for half in range(2):
                cols = s * 64 + half * 32 + g[:, None] * 16 + np.arange(16)[None, :]
                pc[:, j, s, half] = codes[:, rows[:, None], cols]
        for t in range(spans):
            for u in range(4):
                if 4 * t + u < ks:
                    ps[:, j, t, :, u] = scales[:, rows, (4 * t + u) * 2 + g]
    # step-major: K step (scale span) first, then expert, then group
    return pc.transpose(2, 0, 1, 3, 4, 5).reshape(-1), ps.transpose(2, 0, 1, 3, 4).reshape(-1)


@pytest.mark.parametrize("gate_up", [True, False])
def test_pack_weights_layout(ep, gate_up):
    _announce(f"pack weights layout gate_up={gate_up}")
    codes, scales = W.make_mx_weights(77, 2, 128, 320)              # 5 K steps: a ragged last scale span
    pc, ps = ep.pack_moe_weights(to_dev(codes), to_dev(scales), gate_up)
    torch.cuda.synchronize()
    want_c, want_s = _pack_reference(codes, scales, gate_up)
    assert np.array_equal(pc.cpu().numpy(), want_c)
    assert np.array_equal(ps.cpu().numpy(), want_s)
