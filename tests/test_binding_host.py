"""Host-side checks of the Python binding (no GPU needed): every tensor
argument is checked for dtype, shape, contiguity, size and device before its
pointer reaches the library, which can only check pointers and byte counts.

Each case passes CPU tensors that are right in every respect but one; the
binding must name that argument.  A case that is right in every respect
fails on the device check (CPU tensors are never valid), so no case reaches
the library.
"""

import pytest
import torch

T, K, H, E = 4, 2, 256, 8


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _handle(ep):
    h = ep.ep_handle_t()
    h.num_tokens, h.num_max_tokens, h.max_rows = T, 8, 8 * K
    h.num_topk, h.num_experts = K, E
    h.row_align, h.expert_capacity = 1, 0
    return h


def _combine_args():
    return dict(expert_out=torch.zeros(16 * H * 2, dtype=torch.uint8),
                topk_idx=torch.zeros((T, K), dtype=torch.int64),
                topk_weights=torch.zeros((T, K), dtype=torch.float32),
                out=torch.zeros((T, H), dtype=torch.bfloat16))


def _raises(ep, fn, name):
    with pytest.raises(ep.EpError) as ei:
        fn()
    assert ei.value.code == ep.EP_ERR_INVALID_ARG
    assert name in str(ei.value), str(ei.value)


COMBINE_BAD = [
    ("topk_weights", dict(topk_weights=torch.zeros((T, K), dtype=torch.bfloat16))),
    ("topk_weights", dict(topk_weights=torch.zeros((T, K + 1), dtype=torch.float32))),
    ("topk_weights", dict(topk_weights=torch.zeros((K, T), dtype=torch.float32).t())),
    ("out", dict(out=torch.zeros((T, H), dtype=torch.float32))),
    ("out", dict(out=torch.zeros((T, H // 2), dtype=torch.bfloat16))),
    ("out", dict(out=torch.zeros((H, T), dtype=torch.bfloat16).t())),
    ("topk_idx", dict(topk_idx=torch.zeros((T, K + 1), dtype=torch.int64))),
    ("topk_idx", dict(topk_idx=torch.zeros((T, K), dtype=torch.float32))),
    ("topk_idx", dict(topk_idx=torch.zeros(T * K, dtype=torch.int64))),
    ("topk_idx", dict(topk_idx=torch.zeros((K, T), dtype=torch.int64).t())),
    ("GPU tensor", dict()),                                   # all right, but on the CPU
]


@pytest.mark.parametrize("name,kw", COMBINE_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(COMBINE_BAD)])
def test_combine_checks(ep, name, kw):
    a = _combine_args()
    a.update(kw)
    _raises(ep, lambda: ep.ep_combine(_handle(ep), a["expert_out"], "none", H, a["topk_idx"], a["topk_weights"],
                                      a["out"]), name)


def test_combine_raw_idx_needs_dtype(ep):
    a = _combine_args()
    _raises(ep, lambda: ep.ep_combine(_handle(ep), a["expert_out"], "none", H, 1 << 40, a["topk_weights"], a["out"]),
            "idx_dtype")


DISPATCH_BAD = [
    ("x", dict(x=torch.zeros((T, H), dtype=torch.float32))),
    ("x", dict(x=torch.zeros((T + 1, H), dtype=torch.bfloat16))),
    ("x", dict(x=torch.zeros((H, T), dtype=torch.bfloat16).t())),
    ("topk_weights", dict(topk_weights=torch.zeros((T, K), dtype=torch.float64))),
    ("topk_weights", dict(topk_weights=torch.zeros((T - 1, K), dtype=torch.float32))),
    ("recv_weights", dict(recv_weights=torch.zeros(8 * K - 1, dtype=torch.float32))),
    ("recv_weights", dict(recv_weights=torch.zeros(8 * K, dtype=torch.bfloat16))),
    ("GPU tensor", dict()),
]


@pytest.mark.parametrize("name,kw", DISPATCH_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(DISPATCH_BAD)])
def test_dispatch_checks(ep, name, kw):
    a = dict(x=torch.zeros((T, H), dtype=torch.bfloat16), recv=torch.zeros(1 << 16, dtype=torch.uint8),
             topk_weights=torch.zeros((T, K), dtype=torch.float32),
             recv_weights=torch.zeros(8 * K, dtype=torch.float32))
    a.update(kw)
    _raises(ep, lambda: ep.ep_dispatch(_handle(ep), a["x"], H, "mxfp8", a["recv"], a["topk_weights"],
                                       a["recv_weights"]), name)


LAYOUT_BAD = [
    ("recv_count", dict(recv_count=torch.zeros(E, dtype=torch.int32))),
    ("recv_count", dict(recv_count=torch.zeros(E - 1, dtype=torch.int64))),
    ("cumulative_recv_stats", dict(cum=torch.zeros(E, dtype=torch.int64))),
    ("cumulative_recv_stats", dict(cum=torch.zeros(E - 2, dtype=torch.int32))),
    ("topk_idx", dict(topk_idx=torch.zeros((T, K), dtype=torch.int16))),
    ("topk_idx", dict()),                                     # right dtype and shape, on the CPU
]


@pytest.mark.parametrize("name,kw", LAYOUT_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(LAYOUT_BAD)])
@pytest.mark.parametrize("call", ["ep_layout", "ep_layout_dispatch"])
def test_layout_checks(ep, name, kw, call):
    a = dict(topk_idx=torch.zeros((T, K), dtype=torch.int64), recv_count=torch.zeros(E, dtype=torch.int64),
             ws=torch.zeros(1 << 16, dtype=torch.uint8), cum=None)
    a.update(kw)
    if call == "ep_layout":
        fn = lambda: ep.ep_layout(a["topk_idx"], E, 8, a["recv_count"], a["ws"], a["cum"])  # noqa: E731
    else:
        fn = lambda: ep.ep_layout_dispatch(a["topk_idx"], E, 8, a["recv_count"], a["ws"],  # noqa: E731
                                           torch.zeros((T, H), dtype=torch.bfloat16), H, "mxfp8",
                                           torch.zeros(1 << 16, dtype=torch.uint8), cumulative_recv_stats=a["cum"])
    _raises(ep, fn, name)


def test_layout_dispatch_checks_dispatch_args(ep):
    """The one-call layout + dispatch checks its dispatch arguments too (here
    a float32 x) before anything reaches the library."""
    idx = torch.zeros((T, K), dtype=torch.int64)
    _raises(ep, lambda: ep.ep_layout_dispatch(idx, E, 8, torch.zeros(E, dtype=torch.int64),
                                              torch.zeros(1 << 16, dtype=torch.uint8),
                                              torch.zeros((T, H), dtype=torch.float32), H, "mxfp8",
                                              torch.zeros(1 << 16, dtype=torch.uint8)), "x")


def test_backward_checks(ep):
    g = torch.zeros((T, H), dtype=torch.float32)
    _raises(ep, lambda: ep.ep_combine_backward(_handle(ep), g, H, "mxfp8", torch.zeros(1 << 16, dtype=torch.uint8)),
            "grad_out")
    g = torch.zeros((T, H), dtype=torch.bfloat16)
    _raises(ep, lambda: ep.ep_combine_backward(_handle(ep), g, H, "mxfp8", torch.zeros(1 << 16, dtype=torch.uint8),
                                               torch.zeros((T, K + 1), dtype=torch.float32)), "topk_weights")


def test_low_latency_wrappers_check_inputs(ep):
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    idx = torch.zeros((T, K), dtype=torch.int64)
    _raises(ep, lambda: ep.low_latency_dispatch(x, idx, 8, E), "GPU tensor")
    _raises(ep, lambda: ep.low_latency_dispatch(x.float(), idx, 8, E), "x must be")


def _gmm_args(ep, experts, inter=64, hidden=H):
    cb, sb = ep.ep_moe_packed_bytes(experts, 2 * inter, hidden)
    return torch.zeros(cb, dtype=torch.uint8), torch.zeros(sb, dtype=torch.uint8)


GMM_BAD = [
    ("w1", lambda ep: (_gmm_args(ep, E + 1)[0], _gmm_args(ep, E)[1])),       # packed for other experts
    ("w1_scales", lambda ep: (_gmm_args(ep, E)[0], _gmm_args(ep, E - 1)[1])),
    ("w1", lambda ep: (_gmm_args(ep, E)[0].view(torch.int8), _gmm_args(ep, E)[1])),
    ("w1", lambda ep: (_gmm_args(ep, E)[0].view(2, -1), _gmm_args(ep, E)[1])),
    ("GPU tensor", lambda ep: _gmm_args(ep, E)),                            # all right, but on the CPU
]


@pytest.mark.parametrize("name,make", GMM_BAD, ids=[f"{n}-{i}" for i, (n, _) in enumerate(GMM_BAD)])
def test_gmm1_checks_packed_weights(ep, name, make):
    """Packed weights must be exactly what ep_moe_pack_weights fills for the
    handle's experts: the step-major packing puts expert e's fragments of K
    step s at a place that depends on the expert count."""
    w1, w1s = make(ep)
    buf = torch.zeros(1 << 16, dtype=torch.uint8)
    _raises(ep, lambda: ep.ep_moe_gmm1(_handle(ep), buf, H, 64, w1, w1s, "mxfp8", buf), name)


def test_gmm2_checks_packed_weights(ep):
    cb, sb = ep.ep_moe_packed_bytes(E + 2, H, 128)
    buf = torch.zeros(1 << 16, dtype=torch.uint8)
    _raises(ep, lambda: ep.ep_moe_gmm2(_handle(ep), buf, 128, H, torch.zeros(cb, dtype=torch.uint8),
                                       torch.zeros(sb, dtype=torch.uint8), buf), "w2")
