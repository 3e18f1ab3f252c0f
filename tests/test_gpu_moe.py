"""GPU parity of the expert MLP (ep_moe_gmm1 / ep_moe_gmm2) against the
float64 oracle, on the same seeded inputs.

The matrix cores sum each 64-product block with less than float32 precision
(about 3e-4 of the block's sum of |products|), so the bars are bounds, not
bit equality:

* GMM1 with bf16 output: |gpu - a| <= c (|silu'(g)| |u| S_g + |silu(g)| S_u)
  + one bf16 rounding, per element, with S = sum |x w| of the dot product and
  c = MFMA_REL;
* GMM1 with MXFP8 output: the requant rounds a value that can differ from
  the oracle's by the bound above, so each dequantised value lies within that
  bound plus one e4m3 step of the oracle's (blocks whose shared exponents
  differ by one: 25 %), at most 2 % of the codes differ and scale bytes are
  equal or off by one;
* GMM2 on shared synthetic MXFP8 input: |gpu - y| <= c S + one bf16 rounding;
* the whole path (dispatch, GMM1, requant, GMM2, combine): per output row
  ||gpu - oracle|| / ||oracle|| <= 3e-2.

Rows holding no pair are never written (their canaries survive).
"""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from combine_topk_idx_amd import workloads as W
from oracle import codecs, combine as OC, dispatch as OD, moe as OM
from tests.hip_path import DEV, canary_buffer, sample_tokens, to_dev, NAN_BF16
from tests.moe_path import MFMA_REL, gpu_moe, oracle_moe, read_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _bf16_rows(buf, rows, width):
    return buf[: rows * width * 2].view(torch.int16).view(rows, width).cpu().numpy().view(np.uint16)


def _gmm1_bound(rb_data, rb_scales, w1c, w1s, a, rounding=2.0 ** -8):
    xv = OM.mx_dequant(rb_data, rb_scales)
    wv = OM.mx_dequant(w1c, w1s)
    inter = wv.shape[0] // 2
    g, u = xv @ wv[:inter].T, xv @ wv[inter:].T
    S = np.abs(xv) @ np.abs(wv).T
    sg, su = S[:, :inter], S[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    # matrix-core error through silu(g) * u, float32 evaluation of silu, then
    # the output rounding (bf16: 2^-8 relative with margin)
    return MFMA_REL * (dsilu * np.abs(u) * sg + np.abs(OM.silu(g)) * su) + (rounding + 1e-6) * np.abs(a) + 1e-30


def _check_gmm1_bf16(got_bits, a, bound):
    got = codecs.bf16_bits_to_f32(got_bits).astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.abs(got - a)
    assert np.all(err <= bound), f"worst err/bound {np.max(err / bound):.3g}"


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
        bound = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"])
        _check_gmm1_bf16(got[rows], ent["a"], bound)
    free = np.nonzero(lay.row_src < 0)[0]
    assert np.all(got[free] == NAN_BF16)                             # never written


def _check_requant(got_codes, got_scales, want_codes, want_scales, abound, frac=0.02):
    """Codes and scale bytes of a requant whose float32 input differs from the
    oracle's by at most `abound` (the GMM1 bound): scale bytes equal or off by
    one (in at most 1 % of the blocks); rounding moves a value by at most one
    e4m3 step, so in blocks with equal scales |gpu - oracle| <= abound + one
    step; in blocks whose scales differ (amax on either side of a power of
    two) the MX rule saturates the block maximum at 448 under the smaller
    exponent (up to 1/8 below 512), so there the allowance is 25 %."""
    sc_diff = got_scales.astype(int) - want_scales.astype(int)
    assert np.all(np.abs(sc_diff) <= 1)
    assert np.mean(sc_diff != 0) <= 0.01
    gv = OM.mx_dequant(got_codes, got_scales)
    wv = OM.mx_dequant(want_codes, want_scales)
    diff = got_codes != want_codes
    assert np.mean(diff) <= frac, f"{np.mean(diff):.4f} of the codes differ"
    same = np.repeat(sc_diff == 0, 32, axis=-1)
    big = np.maximum(np.abs(gv), np.abs(wv))
    sub = 2.0 ** -9 * np.repeat(codecs.e8m0_decode(np.maximum(got_scales, want_scales)), 32, axis=-1)
    step = np.maximum(big * 2.0 ** -3, sub) * (1 + 1e-9) + abound
    loose = np.maximum(big * 0.25, sub) + abound
    bad = (same & (np.abs(gv - wv) > step)) | (~same & (np.abs(gv - wv) > loose))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} values too far apart; first at {tuple(i)}: gpu {gv[tuple(i)]} "
                             f"oracle {wv[tuple(i)]} (codes {got_codes[tuple(i)]:#x} / {want_codes[tuple(i)]:#x}, "
                             f"scales {got_scales[i[0], i[1] // 32]} / {want_scales[i[0], i[1] // 32]})")
    return float(np.mean(diff))


def test_gmm1_mxfp8_small(ep):
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("gmm1 mxfp8 moe_small")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp, out_quant="mxfp8", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="mxfp8")
    total, off = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    buf = res["a"][:total].cpu().numpy()
    got = OD.RecvBuffer.from_bytes(buf, lay.max_rows, w.I, "mxfp8", lay.num_rows)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        f = _check_requant(got.data[rows], got.scales[rows], ent["q"], ent["qs"], ab)
        print(f"expert {e}: {f:.4f} of the codes differ")


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
    got = codecs.bf16_bits_to_f32(_bf16_rows(y, rows, w.H)).astype(np.float64)
    rc = res["rc"].cpu().numpy()
    _, offs = read_slots(ep, res, w)
    for e in range(w.E_local):
        r = np.arange(offs[e], offs[e] + rc[e])
        if r.size == 0:
            continue
        _, yv = OM.gmm2_rows(ac[0][r], asc[0][r], inp["w2_codes"][e], inp["w2_scales"][e])
        S = OM.abs_products(ac[0][r], asc[0][r], inp["w2_codes"][e], inp["w2_scales"][e])
        bound = MFMA_REL * S + 2.0 ** -8 * np.abs(yv) + 1e-30
        err = np.abs(got[r] - yv)
        assert np.all(err <= bound), f"expert {e}: worst err/bound {np.max(err / bound):.3g}"


def _check_end_to_end(got_bits, want_bits, tol=3e-2):
    got = codecs.bf16_bits_to_f32(got_bits).astype(np.float64)
    want = codecs.bf16_bits_to_f32(want_bits).astype(np.float64)
    assert np.all(np.isfinite(got))
    num = np.linalg.norm(got - want, axis=1)
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-30)
    rel = num / den
    routed = np.linalg.norm(want, axis=1) > 0
    assert np.all(rel[routed] <= tol), f"worst row rel err {np.max(rel[routed]):.3g}"
    assert np.all(got[~routed] == 0)
    return float(np.max(rel[routed])) if routed.any() else 0.0


def test_end_to_end_small(ep):
    w = W.MOE_WORKLOADS["moe_small"]
    _announce("moe end to end, moe_small")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    worst = _check_end_to_end(res["out"], out)
    print(f"worst row relative error {worst:.3g}")


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
            bound = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"])
            _check_gmm1_bf16(got[rows], ent["a"], bound)
        free = np.nonzero(lay.row_src < 0)[0]
        assert np.all(got[free] == NAN_BF16)


def test_mixed_tile_widths(ep):
    """A launch with both tile widths (on a 256-CU device): GMM1 of I = 3072
    has 96 four-group or 64 six-group tiles per chunk; with three chunks the
    six-group plan fits one round and the chunk with the most fragments moves
    to four-group tiles.  Expert 0 has 200 rows, a full 160-row chunk (five
    fragments: narrow) and a 40-row one (two fragments: wide); expert 1 has
    60 rows (wide).  bf16 and MXFP8 outputs against the oracle."""
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
        bound = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"])
        _check_gmm1_bf16(got[rows], ent["a"], bound)
    res = gpu_moe(ep, w, inp, out_quant="mxfp8", stop_after="gmm1")
    lay, rb, per, _ = oracle_moe(w, inp, out_mode="mxfp8")
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    for e, (rows, ent) in enumerate(per):
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        _check_requant(a.data[rows], a.scales[rows], ent["q"], ent["qs"], ab)


def test_capacity_padded_blocks(ep):
    """The [E, C, ...] receive shape of the low-latency API: every expert
    block has C rows, the hot expert's pairs past the C-th are dropped (slot
    -1, never multiplied), the rest of each block is never written; the
    whole path through combine."""
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
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        _check_requant(a.data[rows], a.scales[rows], ent["q"], ent["qs"], ab)
    y = _bf16_rows(res["y"], lay.max_rows, w.H)
    free = np.nonzero(lay.row_src < 0)[0]
    assert free.size > 0 and np.all(y[free] == NAN_BF16)          # padding rows never written
    # GMM2 against the exact products of the GPU's own requantised rows, then
    # combine against the oracle's combine of the GPU's own expert rows (the
    # requant may move a value by one e4m3 step, checked above; with few
    # pairs per token and I = 128 one such step can show in a whole row)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        gv = OM.mx_dequant(a.data[rows], a.scales[rows])
        wv = OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e])
        want = gv @ wv.T
        bound = MFMA_REL * (np.abs(gv) @ np.abs(wv).T) + 2.0 ** -8 * np.abs(want) + 1e-30
        got = codecs.bf16_bits_to_f32(y[rows]).astype(np.float64)
        assert np.all(np.abs(got - want) <= bound), f"expert {e}: GMM2 outside its bound"
    cin = OD.RecvBuffer("none", w.H, lay.num_rows, y.view(np.uint8), np.zeros((lay.max_rows, 0), np.uint8), None)
    assert np.array_equal(res["out"], OC.combine(cin, lay, inp["topk_weights"]))


def test_share_full_size_sampled(ep):
    """The 1024-token, 6-local-expert share at full size (hidden 7168,
    intermediate 3072), sampled tokens through the whole path."""
    w = W.MOE_WORKLOADS["moe_share"]
    _announce("moe_share full size, sampled tokens")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    toks = sample_tokens(W.Workload("s", w.T, w.H, w.E_local, w.k, "int64", "mxfp8", "uniform"), inp["topk_idx"],
                         n=24)
    lay, rb, per, out = oracle_moe(w, inp, tokens=toks)
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        f = _check_requant(a.data[rows], a.scales[rows], ent["q"], ent["qs"], ab)
        print(f"expert {e}: {f:.4f} of the codes differ")
    worst = _check_end_to_end(res["out"][toks], out)
    print(f"worst row relative error {worst:.3g}")


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
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        _check_requant(a.data[rows], a.scales[rows], ent["q"], ent["qs"], ab, frac=0.05)
    y = _bf16_rows(res["y"], lay.max_rows, w.H)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        got = codecs.bf16_bits_to_f32(y[rows]).astype(np.float64)
        # GMM2 reads the GPU's own requantised rows (checked above against the
        # oracle's), so its exact reference is the dot product with those rows
        gv = OM.mx_dequant(a.data[rows], a.scales[rows])
        wv = OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e])
        want = gv @ wv.T
        S = np.abs(gv) @ np.abs(wv).T
        bound = MFMA_REL * S + 2.0 ** -8 * np.abs(want) + 1e-30
        err = np.abs(got - want)
        assert np.all(err <= bound), f"expert {e}: worst err/bound {np.max(err / bound):.3g}"
    worst = _check_end_to_end(res["out"], out)
    print(f"worst row relative error {worst:.3g}")


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
        bound = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"])
        _check_gmm1_bf16(got[rows], ent["a"], bound)
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
]


@pytest.mark.parametrize("case", FUZZ, ids=[f"f{c[-1]}" for c in FUZZ])
def test_gemm_shapes(ep, case):
    """Assorted shapes through the whole path: GMM1's MXFP8 rows against the
    oracle's requant, GMM2 against the exact product with the GPU's own GMM1
    rows, rows holding no pair never written."""
    T, H, I, Et, El, k, seed = case
    w = W.MoeWorkload(f"fz{seed}", T, H, I, Et, El, k, seed=seed)
    _announce(f"gemm shapes T={T} H={H} I={I} experts {El}/{Et} k={k}")
    inp = W.make_moe_inputs(w)
    res = gpu_moe(ep, w, inp)
    lay, rb, per, out = oracle_moe(w, inp)
    total, _ = ep.ep_buffer_bytes(lay.max_rows, w.I, "mxfp8")
    a = OD.RecvBuffer.from_bytes(res["a"][:total].cpu().numpy(), lay.max_rows, w.I, "mxfp8", lay.num_rows)
    y = _bf16_rows(res["y"], lay.max_rows, w.H)
    for e, (rows, ent) in enumerate(per):
        if ent is None:
            continue
        ab = _gmm1_bound(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e], ent["a"], 0.0)
        _check_requant(a.data[rows], a.scales[rows], ent["q"], ent["qs"], ab, frac=0.05)
        gv = OM.mx_dequant(a.data[rows], a.scales[rows])
        wv = OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e])
        want = gv @ wv.T
        bound = MFMA_REL * (np.abs(gv) @ np.abs(wv).T) + 2.0 ** -8 * np.abs(want) + 1e-30
        err = np.abs(codecs.bf16_bits_to_f32(y[rows]).astype(np.float64) - want)
        assert np.all(err <= bound), f"expert {e}: worst GMM2 err/bound {np.max(err / bound):.3g}"
    free = np.nonzero(lay.row_src < 0)[0]
    assert np.all(y[free] == NAN_BF16)


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
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("gate_up", [True, False])
def test_pack_weights_layout(ep, gate_up):
    _announce(f"pack weights layout gate_up={gate_up}")
    codes, scales = W.make_mx_weights(77, 2, 128, 320)              # 5 K steps: a ragged last scale span
    pc, ps = ep.pack_moe_weights(to_dev(codes), to_dev(scales), gate_up)
    torch.cuda.synchronize()
    want_c, want_s = _pack_reference(codes, scales, gate_up)
    assert np.array_equal(pc.cpu().numpy(), want_c)
    assert np.array_equal(ps.cpu().numpy(), want_s)
