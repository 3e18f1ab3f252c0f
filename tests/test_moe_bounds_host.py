"""Host checks of the expert-MLP bounds (``tests/moe_bounds.py``) that the GPU
tests apply: the oracle's own results pass them, and planted mistakes (a
code flipped where no rounding is ambiguous, a scale byte off by one, a GMM2
row off by a few percent, a combine weight taken from the wrong pair) fail
them.  The float64 e4m3 rounding they use agrees with the oracle's encoder."""

import numpy as np
import pytest

from combine_topk_idx_amd import workloads as W
from oracle import codecs, moe as OM
from tests import moe_bounds as MB
from tests.moe_path import oracle_moe


def test_e4m3_index_matches_the_oracle_encoder():
    rng = np.random.default_rng(3)
    mags = codecs.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float32)
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)     # exact in float32
    v = np.concatenate([mags, -mags, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.inf),
                        rng.standard_normal(20000).astype(np.float32) * 64, np.float32([500, -900, 448, 1e-9])])
    v = np.clip(v, -448, 448).astype(np.float32)
    codes = codecs.e4m3_encode(v)
    want = np.where(codes & 0x80, -(codes & 0x7F).astype(np.int64), (codes & 0x7F).astype(np.int64))
    want = np.where(v == 0, 0, want)
    assert np.array_equal(MB.e4m3_index(v.astype(np.float64)), want)


@pytest.fixture(scope="module")
def small():
    w = W.MOE_WORKLOADS["moe_small"]
    inp = W.make_moe_inputs(w)
    lay, rb, per, out = oracle_moe(w, inp)
    e = next(i for i, (rows, ent) in enumerate(per) if ent is not None)
    rows, ent = per[e]
    xv = OM.mx_dequant(rb.data[rows], rb.scales[rows])
    w1v = OM.mx_dequant(inp["w1_codes"][e], inp["w1_scales"][e])
    w2v = OM.mx_dequant(inp["w2_codes"][e], inp["w2_scales"][e])
    a, B1 = MB.gmm1_bound(xv, w1v)
    return dict(w=w, inp=inp, lay=lay, per=per, out=out, ent=ent, rows=rows, a=a, B1=B1, w2v=w2v)


def test_bound_of_gmm1_covers_float32_rounding(small):
    a, B1 = small["a"], small["B1"]
    assert np.allclose(a, small["ent"]["a"], rtol=1e-12, atol=1e-300)
    assert np.all(np.abs(a.astype(np.float32) - a) <= B1)
    # and is small: below bf16's half step for most elements
    assert np.median(B1 / np.maximum(np.abs(a), 1e-30)) < 2.0 ** -8


def test_requant_check_passes_the_oracle_and_catches_mistakes(small):
    ent, a32, B1 = small["ent"], small["ent"]["a"].astype(np.float32), small["B1"]
    D, st = MB.check_requant(ent["q"], ent["qs"], a32, B1, ent["q"], ent["qs"])
    assert st["differ"] == 0 and st["ambiguous"] < 0.2 * st["codes"]
    se_lo, se_hi, intervals = MB.requant_intervals(a32, B1)
    lo, hi = intervals(ent["qs"].astype(np.int64) - 127)
    r, c = np.argwhere((lo == hi) & (lo > 0) & (lo < 126))[0]
    q = ent["q"].copy()
    q[r, c] += 1                                          # one step up where nothing is ambiguous
    with pytest.raises(AssertionError):
        MB.check_requant(q, ent["qs"], a32, B1, ent["q"], ent["qs"])
    qs = ent["qs"].copy()
    b = np.argwhere(se_lo == se_hi)[0]
    qs[tuple(b)] += 1                                     # a scale byte the block maximum cannot reach
    with pytest.raises(AssertionError):
        MB.check_requant(ent["q"], qs, a32, B1, ent["q"], ent["qs"])


def test_gmm2_and_combine_bounds(small):
    ent, w2v = small["ent"], small["w2v"]
    want_v = OM.mx_dequant(ent["q"], ent["qs"])
    bound, _ = MB.gmm2_bound(want_v, np.zeros_like(want_v), w2v, ent["y"])
    y_bf16 = codecs.bf16_bits_to_f32(codecs.f32_to_bf16_bits(ent["y"].astype(np.float32))).astype(np.float64)
    assert np.all(np.abs(y_bf16 - ent["y"]) <= bound)
    bad = y_bf16.copy()
    i = np.unravel_index(np.argmax(np.abs(ent["y"])), bad.shape)
    bad[i] *= 1.03                                        # a 3 % error in one element
    assert np.abs(bad - ent["y"])[i] > bound[i]
    # combine: the oracle's output passes its own bound; a weight taken from
    # the wrong pair does not
    w, lay, out, inp = small["w"], small["lay"], small["out"], small["inp"]
    y_exact = np.zeros((lay.max_rows, w.H))
    for rows, e in small["per"]:
        if e is not None:
            y_exact[rows] = e["y"]
    rows_bound = 2.0 ** -9 * np.abs(y_exact)
    want = codecs.bf16_bits_to_f32(out).astype(np.float64)
    wts = inp["topk_weights"]
    cb = MB.combine_bound(rows_bound, y_exact, lay.slot, wts, want)
    assert np.all(cb > 0)
    t = np.nonzero((lay.slot >= 0).sum(axis=1) >= 2)[0][0]
    j0, j1 = np.nonzero(lay.slot[t] >= 0)[0][:2]
    wrong = sum(float(wts[t, j1 if j == j0 else j]) * y_exact[lay.slot[t, j]] for j in range(w.k)
                if lay.slot[t, j] >= 0)
    assert np.any(np.abs(wrong - want[t]) > cb[t])
