"""Pins of the oracle's dispatch and combine, and planted-mistake checks.

* dispatch ``none``: every routed receive row equals its token bit for bit;
* combine with unit weights and bf16 rows: out == bf16(k_eff * x) exactly
  (k_eff <= 16 equal terms sum exactly in float32) -- the invariant stated for
  the method; k_eff is counted here directly from topk_idx;
* combine with general weights: within one bf16 ulp of the float64 sum
  rounded once, plus the float32 accumulation bound;
* quantised round trips within each format's error;
* planted mistakes (wrong order in the layout, weights dropped, fp8 ties away
  from even, a dropped term in combine) are each caught by one of the pins.
"""

import numpy as np
import pytest

from combine_topk_idx_amd import workloads as W
from oracle import codecs, combine as C, dispatch as D, layout as L, quant as Q


def _case(seed, T=40, H=96, E=6, k=4, neg=0.2, mode="none"):
    w = W.random_workload(seed, T, H, E, k, mode, neg_frac=neg)
    inp = W.make_inputs(w)
    return w, inp


@pytest.mark.parametrize("seed", range(4))
def test_dispatch_none_copies_rows(seed):
    w, inp = _case(seed)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    rb = D.dispatch(inp["x"], lay, "none", inp["topk_weights"])
    for t in range(w.T):
        for j in range(w.k):
            r = lay.slot[t, j]
            if r >= 0:
                assert np.array_equal(rb.data[r].view(np.uint16), inp["x"][t])
                assert rb.weights[r] == inp["topk_weights"][t, j]


def _keff(idx, E):
    return ((idx >= 0) & (idx < E)).sum(axis=1)


@pytest.mark.parametrize("seed", range(4))
def test_combine_unit_weights_is_keff_times_x(seed):
    w, inp = _case(seed, k=16, E=5, neg=0.3)
    idx = inp["topk_idx"]
    if seed == 3:
        idx = W.with_duplicates(idx, seed)
    lay = L.layout(idx, w.E, w.T)
    rb = D.dispatch(inp["x"], lay, "none")
    out = C.combine(rb, lay, np.ones((w.T, w.k), np.float32))
    keff = _keff(idx, w.E).astype(np.float64)
    ref = W.bf16_from_f32((codecs.bf16_bits_to_f32(inp["x"]).astype(np.float64) * keff[:, None]).astype(np.float32))
    # k_eff * x is exact in float64 and float32 (8-bit mantissa times <= 16)
    assert np.array_equal(out, ref)
    assert np.all(out[keff == 0] == 0)               # +0 rows


@pytest.mark.parametrize("seed", range(4))
def test_combine_general_weights_within_one_ulp(seed):
    w, inp = _case(seed, T=30, H=128, E=7, k=8, neg=0.1)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    y = W.make_expert_out(w)
    rb = D.RecvBuffer("none", w.H, lay.num_rows, y.view(np.uint8).reshape(w.max_rows, -1),
                      np.zeros((w.max_rows, 0), np.uint8), None)
    out = codecs.bf16_bits_to_f32(C.combine(rb, lay, inp["topk_weights"])).astype(np.float64)
    yf = codecs.bf16_bits_to_f32(y).astype(np.float64)
    ref = np.zeros((w.T, w.H))
    mag = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            r = lay.slot[t, j]
            if r >= 0:
                p = float(inp["topk_weights"][t, j]) * yf[r]
                ref[t] += p
                mag[t] += np.abs(p)
    ref_bf = codecs.bf16_bits_to_f32(codecs.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    ulp = np.maximum(np.abs(ref_bf), 2.0 ** -126) * 2.0 ** -7
    # float32: one rounding per product and per add, at most 2k of them
    acc_err = 2 * w.k * 2.0 ** -24 * mag
    assert np.all(np.abs(out - ref) <= ulp + acc_err)


@pytest.mark.parametrize("mode,rel", [("int8_token", 0.02), ("fp8_b128", 0.04),
                                      ("mxfp8", 0.05), ("mxfp4", 0.2),
                                      ("fp8_b128_pow2", 0.05), ("fp8_b128_ue8m0", 0.05)])
def test_dispatch_combine_quantised_roundtrip(mode, rel):
    w, inp = _case(5, T=24, H=256, E=8, k=3, neg=0.0, mode=mode)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    rb = D.dispatch(inp["x"], lay, mode)
    ones = np.ones((w.T, w.k), np.float32) / w.k
    out = codecs.bf16_bits_to_f32(C.combine(rb, lay, ones)).astype(np.float64)
    xf = codecs.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    assert np.linalg.norm(out - xf) / np.linalg.norm(xf) < rel


def test_buffer_bytes_layout():
    total, off = D.buffer_bytes(10, 7168, "mxfp4")
    assert off == D.align_up(10 * 3584, 256) and total == off + 10 * 224
    total, off = D.buffer_bytes(3, 32, "int8_token")
    assert off == 256 and total == 256 + 12


def test_ue8m0_and_pow2_buffers_decode_alike():
    """The two power-of-two scale stores hold the same codes and the same
    scale values, so combine gives the same bits from either."""
    w, inp = _case(11, T=16, H=256, E=4, k=2, mode="fp8_b128_pow2")
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    a = D.dispatch(inp["x"], lay, "fp8_b128_pow2")
    b = D.dispatch(inp["x"], lay, "fp8_b128_ue8m0")
    assert np.array_equal(a.data, b.data)
    assert a.scales.shape[1] == 4 * b.scales.shape[1]
    assert np.array_equal(C.combine(a, lay, inp["topk_weights"]), C.combine(b, lay, inp["topk_weights"]))


def test_interleaved_buffer_worked_example():
    # 2 rows, H = 32, mxfp8: 32 data bytes + 1 scale byte -> one 128-byte line per row
    data = np.arange(64, dtype=np.uint8).reshape(2, 32)
    scales = np.array([[200], [201]], np.uint8)
    rb = D.RecvBuffer("mxfp8", 32, 2, data, scales, None)
    buf = rb.to_bytes(interleaved=True)
    assert buf.size == 256 and D.buffer_bytes(2, 32, "mxfp8", True) == (256, 32)
    assert buf[:32].tolist() == list(range(32)) and buf[32] == 200 and not buf[33:128].any()
    assert buf[128:160].tolist() == list(range(32, 64)) and buf[160] == 201 and not buf[161:].any()
    # int8 per token at H = 64: 64 + 4 bytes -> 128; the float32 scale sits right after the codes
    assert D.interleaved_stride(64, "int8_token") == 128
    assert D.interleaved_stride(7168, "fp8_b128") == 7424          # 7168 + 224 = 7392 -> 58 lines
    assert D.interleaved_stride(7168, "mxfp4") == 3840             # 3584 + 224 = 3808 -> 30 lines
    assert D.interleaved_stride(7168, "fp8_b128_ue8m0") == 7296    # 7168 + 56 -> 57 lines
    assert D.interleaved_stride(256, "none") == 512


@pytest.mark.parametrize("mode", ["int8_token", "fp8_b128", "mxfp8", "mxfp4", "fp8_b128_ue8m0", "none"])
def test_interleaved_roundtrip(mode):
    w, inp = _case(12, T=9, H=384, E=4, k=2, mode=mode)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    rb = D.dispatch(inp["x"], lay, mode)
    buf = rb.to_bytes(interleaved=True)
    rb2 = D.RecvBuffer.from_bytes(buf, w.max_rows, w.H, mode, rb.num_rows, interleaved=True)
    assert np.array_equal(rb.data, rb2.data) and np.array_equal(rb.scales, rb2.scales)
    # the same rows, region form
    rb3 = D.RecvBuffer.from_bytes(rb.to_bytes(), w.max_rows, w.H, mode, rb.num_rows)
    assert np.array_equal(rb3.data, rb2.data) and np.array_equal(rb3.scales, rb2.scales)


def test_recv_buffer_bytes_roundtrip():
    w, inp = _case(9, T=10, H=64, E=4, k=2, mode="mxfp8")
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    rb = D.dispatch(inp["x"], lay, "mxfp8")
    rb2 = D.RecvBuffer.from_bytes(rb.to_bytes(), w.max_rows, w.H, "mxfp8", rb.num_rows)
    assert np.array_equal(rb.data, rb2.data) and np.array_equal(rb.scales, rb2.scales)


# ---------------------------------------------------------------------------
# planted mistakes: each must trip one of the pins above
# ---------------------------------------------------------------------------


def test_planted_unstable_layout_is_caught(monkeypatch):
    from tests.test_oracle_layout import _brute
    rng = np.random.default_rng(0)
    idx = rng.integers(-1, 5, size=(30, 4))
    real = L.layout

    def reversed_order(topk_idx, E, tmax, cum_stats=None):
        lay = real(topk_idx[::-1].copy(), E, tmax)   # assigns rows from the last token
        return lay

    cnt, rows = _brute(idx, 5)
    bad = reversed_order(idx, 5, 30)
    assert not np.array_equal(bad.row_src[:bad.num_rows], rows)


def test_planted_dropped_weight_is_caught():
    w, inp = _case(1, T=30, H=128, E=7, k=8, neg=0.1)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    y = W.make_expert_out(w)
    rb = D.RecvBuffer("none", w.H, lay.num_rows, y.view(np.uint8).reshape(w.max_rows, -1),
                      np.zeros((w.max_rows, 0), np.uint8), None)
    wrong = C.combine(rb, lay, np.ones_like(inp["topk_weights"]))   # weights ignored
    right = C.combine(rb, lay, inp["topk_weights"])
    assert not np.array_equal(wrong, right)


def test_planted_ties_away_is_caught():
    # rounding half away from zero instead of half to even disagrees with torch
    mids = ((codecs.E4M3_POS_VALUES[:-1] + codecs.E4M3_POS_VALUES[1:]) / 2).astype(np.float32)
    hi = np.searchsorted(codecs.E4M3_POS_VALUES, mids)
    away = hi.astype(np.uint8)
    import torch
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(away, ref)
    assert np.array_equal(codecs.e4m3_encode(mids), ref)


def test_planted_dropped_term_is_caught(monkeypatch):
    w, inp = _case(2, k=16, E=5, neg=0.0)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    rb = D.dispatch(inp["x"], lay, "none")
    real = C.combine_token

    def drop_last(expert_out, lay_, wts, t):
        s = lay_.slot.copy()
        s[t, -1] = -1
        return real(expert_out, L.Layout(lay_.num_tokens, lay_.num_topk, lay_.num_experts,
                                         lay_.max_rows, lay_.count, lay_.offsets, s,
                                         lay_.row_src, lay_.status), wts, t)

    monkeypatch.setattr(C, "combine_token", drop_last)
    out = C.combine(rb, lay, np.ones((w.T, w.k), np.float32))
    keff = _keff(inp["topk_idx"], w.E).astype(np.float64)
    ref = W.bf16_from_f32((codecs.bf16_bits_to_f32(inp["x"]).astype(np.float64) * keff[:, None]).astype(np.float32))
    assert not np.array_equal(out, ref)


@pytest.mark.parametrize("mode", ["mxfp4", "fp8_b128", "int8_token"])
def test_parallel_dispatch_helper_is_the_oracle_dispatch(mode):
    """tests/oracle_pool.dispatch_parallel (the full-size GPU tests' expected
    receive rows, quantised in worker processes) returns exactly the oracle's
    dispatch: same codes and scales in every row, same defined rows."""
    from tests.oracle_pool import dispatch_parallel
    w = W.random_workload(77, 300, 256, 16, 4, mode, neg_frac=0.2)
    inp = W.make_inputs(w)
    lay = L.layout(inp["topk_idx"], w.E, w.T)
    want = D.dispatch(inp["x"], lay, mode)
    got = dispatch_parallel(inp["x"], lay, mode, workers=2)
    assert got.num_rows == want.num_rows
    assert np.array_equal(got.data, want.data) and np.array_equal(got.scales, want.scales)
