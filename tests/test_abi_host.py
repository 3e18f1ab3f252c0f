"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function ``include/ep.h`` declares;
* every argument rule returns its documented error code before anything is
  launched (fake, well-aligned device addresses are passed; a call that got
  past validation would try to launch and fail differently);
* the same rules, asked of the oracle's ``validate``, raise where the ABI
  fails and pass where it passes;
* size queries agree with the oracle's buffer layout.
"""

import ctypes
import os
import re

import pytest

from oracle import dispatch as OD, validate as OV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ep():
    from combine_topk_idx_amd import ep as _ep
    return _ep


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ep.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ep_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(ep):
    names = _declared_functions()
    assert set(names) == set(ep.SYMBOLS)
    lib = ctypes.CDLL(ep.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(ep):
    """The built library reports the version its header declares (4: the
    packed expert weights became step-major)."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ep.h")).read()
    declared = int(re.search(r"#define EP_ABI_VERSION (\d+)", hdr).group(1))
    assert declared == 4
    assert ep.ep_abi_version() == declared


FAKE = 1 << 40          # 256-byte aligned, never dereferenced on the host


def _layout(ep, *, idx=FAKE, dtype=1, T=4, k=2, tmax=8, E=8, rc=FAKE, cum=None, ws=FAKE, wsb=1 << 30,
            handle=True):
    h = ep.ep_handle_t()
    return ep._lib.ep_layout(idx, dtype, T, k, tmax, E, rc, cum, ws, wsb,
                             ctypes.byref(h) if handle else None, None)


LAYOUT_BAD = [
    (dict(dtype=2), 1), (dict(k=0), 1), (dict(k=17), 1), (dict(E=0), 1), (dict(E=513), 1),
    (dict(T=-1), 1), (dict(T=9), 1), (dict(tmax=(1 << 31) // 2), 1), (dict(idx=None), 1),
    (dict(idx=FAKE + 4), 1), (dict(idx=FAKE + 4, dtype=0), None), (dict(rc=None), 1), (dict(rc=FAKE + 4), 1),
    (dict(cum=FAKE + 2), 1), (dict(ws=None), 1), (dict(ws=FAKE + 16), 1), (dict(wsb=100), 3),
    (dict(handle=False), 1),
]


@pytest.mark.parametrize("kw,code", LAYOUT_BAD)
def test_layout_rejects(ep, kw, code):
    if code is None:
        pytest.skip("valid arguments (int32 ids need only 4-byte alignment): would launch")
    assert _layout(ep, **kw) == code
    assert ep.ep_last_error().startswith("ep_layout")


@pytest.mark.parametrize("kw,code", LAYOUT_BAD)
def test_oracle_validate_agrees_on_layout_limits(kw, code):
    keys = {"k", "E", "T", "tmax"}
    if code is None or not set(kw) <= keys:
        pytest.skip("pointer / dtype / buffer checks have no oracle counterpart")
    a = dict(T=4, k=2, tmax=8, E=8)
    a.update(kw)
    with pytest.raises(ValueError):
        OV.check_layout(a["T"], a["k"], a["tmax"], a["E"])


def test_oracle_validate_accepts_defaults():
    OV.check_layout(4, 2, 8, 8)
    OV.check_layout(0, 16, 0, 512)
    for m in OV.QUANT_MODES:
        OV.check_hidden(7168, m)


def _layout_ex(ep, align=1, cap=0, tmax=8, k=2, E=8, wsb=1 << 30):
    h = ep.ep_handle_t()
    return ep._lib.ep_layout_ex(FAKE, 1, 4, k, tmax, E, align, cap, FAKE, None, FAKE, wsb, ctypes.byref(h), None)


LAYOUT_EX_BAD = [
    (dict(align=0), 1), (dict(align=1025), 1), (dict(cap=-1), 1), (dict(align=2, cap=4), 1),
    (dict(cap=1 << 23, E=512), 1), (dict(tmax=(1 << 30) - 1, align=1024), 1), (dict(align=64, wsb=64), 3),
]


@pytest.mark.parametrize("kw,code", LAYOUT_EX_BAD)
def test_layout_ex_rejects(ep, kw, code):
    assert _layout_ex(ep, **kw) == code
    assert ep.ep_last_error().startswith("ep_layout_ex")


@pytest.mark.parametrize("kw,code", LAYOUT_EX_BAD)
def test_oracle_validate_agrees_on_padding_limits(kw, code):
    if "wsb" in kw:
        pytest.skip("buffer-size check has no oracle counterpart")
    a = dict(align=1, cap=0, tmax=8, k=2, E=8)
    a.update(kw)
    with pytest.raises(ValueError):
        OV.check_padding(a["k"], a["tmax"], a["E"], a["align"], a["cap"])


@pytest.mark.parametrize("tmax,k,E,align,cap", [(8, 2, 8, 1, 0), (100, 8, 256, 128, 0), (100, 8, 256, 1, 100),
                                                (0, 1, 1, 7, 0), (16384, 8, 256, 1, 16384), (3, 16, 512, 1024, 0)])
def test_layout_rows_matches_oracle(ep, tmax, k, E, align, cap):
    from oracle import layout as OL
    import numpy as np
    rows = ep.ep_layout_rows(tmax, k, E, align, cap)
    assert rows == OV.check_padding(k, tmax, E, align, cap)
    if tmax * k <= 4096:
        lay = OL.layout(np.zeros((0, k), np.int64), E, tmax, row_align=align, expert_capacity=cap)
        assert lay.max_rows == rows
    assert ep.ep_workspace_bytes_ex(tmax, k, E, align, cap) >= 4 * rows
    if align == 1 and cap == 0:
        assert ep.ep_workspace_bytes_ex(tmax, k, E, 1, 0) == ep.ep_workspace_bytes(tmax, k, E)


def test_layout_rows_rejects(ep):
    assert ep.ep_layout_rows(8, 2, 8, 0, 0) == -1
    assert ep.ep_layout_rows(8, 2, 8, 2, 3) == -1
    assert ep.ep_layout_rows(8, 0, 8, 1, 0) == -1
    assert ep.ep_workspace_bytes_ex(8, 2, 8, 1, -2) == 0


def _handle(ep, T=4, k=2, tmax=8, E=8):
    h = ep.ep_handle_t()
    h.num_tokens, h.num_max_tokens, h.max_rows = T, tmax, tmax * k
    h.num_topk, h.num_experts = k, E
    h.row_align, h.expert_capacity = 1, 0
    h.offsets = h.slot = h.row_src = h.status = FAKE
    return h


DISPATCH_BAD = [
    (dict(hidden=0), 1), (dict(hidden=48), 1), (dict(hidden=96, quant=2), 1), (dict(quant=7), 1),
    (dict(hidden=65568), 2), (dict(x=None), 1), (dict(x=FAKE + 8), 1), (dict(recv=None), 1),
    (dict(recv=FAKE + 8), 1), (dict(recv_bytes=10), 3), (dict(rw=FAKE, w=None), 1), (dict(w=FAKE + 2), 1),
    (dict(h_bad="k"), 1), (dict(h_bad="rows"), 1), (dict(h_bad="ptr"), 1), (dict(h_none=True), 1),
    (dict(h_bad="align"), 1),
]


@pytest.mark.parametrize("kw,code", DISPATCH_BAD)
def test_dispatch_rejects(ep, kw, code):
    h = _handle(ep)
    if kw.get("h_bad") == "k":
        h.num_topk = 17
    elif kw.get("h_bad") == "rows":
        h.max_rows = 3
    elif kw.get("h_bad") == "ptr":
        h.slot = None
    elif kw.get("h_bad") == "align":
        h.row_align = 4             # max_rows no longer matches the arrangement
    hp = None if kw.get("h_none") else ctypes.byref(h)
    hidden = kw.get("hidden", 256)
    quant = kw.get("quant", 3)
    rc = ep._lib.ep_dispatch(hp, kw.get("x", FAKE), hidden, kw.get("w", None), quant, kw.get("recv", FAKE),
                             kw.get("recv_bytes", 1 << 30), kw.get("rw", None), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_dispatch")


# ep_layout_dispatch checks the layout arguments and then the dispatch ones;
# either kind of failure launches nothing and names the call
LAYOUT_DISPATCH_BAD = [
    (dict(dtype=2), 1), (dict(k=17), 1), (dict(E=513), 1), (dict(T=9), 1), (dict(idx=None), 1),
    (dict(rc=None), 1), (dict(ws=FAKE + 16), 1), (dict(wsb=100), 3), (dict(align=2, cap=4), 1),
    (dict(handle=False), 1), (dict(hidden=48), 1), (dict(quant=7), 1), (dict(x=None), 1),
    (dict(x=FAKE + 8), 1), (dict(recv=None), 1), (dict(recv_bytes=10), 3), (dict(rw=FAKE, w=None), 1),
    (dict(w=FAKE + 2), 1),
]


@pytest.mark.parametrize("kw,code", LAYOUT_DISPATCH_BAD)
def test_layout_dispatch_rejects(ep, kw, code):
    h = ep.ep_handle_t()
    rc = ep._lib.ep_layout_dispatch(kw.get("idx", FAKE), kw.get("dtype", 1), kw.get("T", 4), kw.get("k", 2), 8,
                                    kw.get("E", 8), kw.get("align", 1), kw.get("cap", 0), kw.get("rc", FAKE), None,
                                    kw.get("ws", FAKE), kw.get("wsb", 1 << 30), kw.get("x", FAKE),
                                    kw.get("hidden", 256), kw.get("w", None), kw.get("quant", 3),
                                    kw.get("recv", FAKE), kw.get("recv_bytes", 1 << 30), kw.get("rw", None),
                                    None if kw.get("handle") is False else ctypes.byref(h), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_layout_dispatch")


COMBINE_BAD = [
    (dict(hidden=40), 1), (dict(quant=-1), 1), (dict(inp=None), 1), (dict(inp=FAKE + 4), 1),
    (dict(in_bytes=5), 3), (dict(w=None), 1), (dict(out=None), 1), (dict(out=FAKE + 2), 1),
    (dict(hidden=128 + 32, quant=2), 1), (dict(hidden=128 + 64, quant=5), 1), (dict(hidden=96, quant=6), 1),
    (dict(quant=7), 1),
    # topk_idx must be the dispatch ids: present, of a known dtype, aligned to it
    (dict(idx=None), 1), (dict(idx_dtype=2), 1), (dict(idx_dtype=-1), 1), (dict(idx=FAKE + 4), 1),
    (dict(idx=FAKE + 2, idx_dtype=0), 1), (dict(idx=FAKE + 4, idx_dtype=0), None),
]


@pytest.mark.parametrize("kw,code", COMBINE_BAD)
def test_combine_rejects(ep, kw, code):
    if code is None:
        pytest.skip("valid arguments (int32 ids need only 4-byte alignment): would launch")
    h = _handle(ep)
    rc = ep._lib.ep_combine(ctypes.byref(h), kw.get("inp", FAKE), kw.get("in_bytes", 1 << 30),
                            kw.get("quant", 0), kw.get("hidden", 256), kw.get("idx", FAKE), kw.get("idx_dtype", 1),
                            kw.get("w", FAKE), kw.get("out", FAKE), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_combine")


BACKWARD_BAD = [
    (dict(hidden=48), 1), (dict(quant=9), 1), (dict(grad=None), 1), (dict(grad=FAKE + 8), 1),
    (dict(buf=None), 1), (dict(buf=FAKE + 4), 1), (dict(buf_bytes=3), 3), (dict(w=FAKE + 1), 1),
    (dict(hidden=160, quant=2), 1),
]


@pytest.mark.parametrize("kw,code", BACKWARD_BAD)
def test_combine_backward_rejects(ep, kw, code):
    h = _handle(ep)
    rc = ep._lib.ep_combine_backward(ctypes.byref(h), kw.get("grad", FAKE), kw.get("hidden", 256), kw.get("w", None),
                                     kw.get("quant", 3), kw.get("buf", FAKE), kw.get("buf_bytes", 1 << 30), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_combine_backward")


@pytest.mark.parametrize("hidden,mode", [(32, "none"), (7168, "int8_token"), (7168, "fp8_b128"),
                                         (96, "mxfp8"), (7168, "mxfp4"), (1024, "mxfp4"),
                                         (7168, "fp8_b128_pow2"), (7168, "fp8_b128_ue8m0"),
                                         (384, "fp8_b128_ue8m0")])
@pytest.mark.parametrize("rows", [0, 1, 37, 131072])
def test_buffer_bytes_matches_oracle(ep, hidden, mode, rows):
    assert ep.ep_buffer_bytes(rows, hidden, mode) == OD.buffer_bytes(rows, hidden, mode)


@pytest.mark.parametrize("hidden,mode", [(32, "none"), (7168, "int8_token"), (64, "int8_token"),
                                         (7168, "fp8_b128"), (96, "mxfp8"), (7168, "mxfp4"),
                                         (384, "fp8_b128_ue8m0"), (7168, "fp8_b128_pow2")])
@pytest.mark.parametrize("rows", [0, 1, 37, 131072])
def test_interleaved_buffer_bytes_matches_oracle(ep, hidden, mode, rows):
    assert ep.ep_buffer_bytes(rows, hidden, mode, interleaved=True) == OD.buffer_bytes(rows, hidden, mode, True)


def test_quant_flag_bits_rejected(ep):
    for bad in (0x200, 0x101 | 0x400, 0x107):
        with pytest.raises(ep.EpError) as e:
            ep.ep_buffer_bytes(4, 256, bad)
        assert e.value.code == 1


def test_buffer_bytes_rejects(ep):
    with pytest.raises(ep.EpError) as e:
        ep.ep_buffer_bytes(10, 100, "none")
    assert e.value.code == 1
    with pytest.raises(ep.EpError):
        ep.ep_buffer_bytes(-1, 128, "none")
    with pytest.raises(ep.EpError):
        ep.ep_buffer_bytes(1, 96, "fp8_b128")
    for q in ("fp8_b128_pow2", "fp8_b128_ue8m0"):
        with pytest.raises(ep.EpError):
            ep.ep_buffer_bytes(1, 160, q)
        with pytest.raises(ValueError):
            OV.check_hidden(160, q)


def test_workspace_bytes(ep):
    assert ep.ep_workspace_bytes(16384, 8, 256) > 16384 * 8 * 8
    assert ep.ep_workspace_bytes(0, 1, 1) > 0
    assert ep.ep_workspace_bytes(10, 0, 8) == 0
    assert ep.ep_workspace_bytes(10, 17, 8) == 0
    assert ep.ep_workspace_bytes(10, 8, 513) == 0
    assert ep.ep_workspace_bytes(1 << 30, 8, 8) == 0


def test_flag_mapping(ep):
    assert ep.quant_mode(use_fp8=False) == "none"
    assert ep.quant_mode(use_fp8=True) == "int8_token"
    assert ep.quant_mode(use_fp8=True, use_ue8m0=True) == "mxfp8"
    assert ep.quant_mode(use_fp8=True, use_mxfp4=True) == "mxfp4"
    with pytest.raises(ep.EpError):
        ep.quant_mode(use_fp8=False, use_ue8m0=True)
    assert ep.quant_mode(use_fp8=True, use_ue8m0=True, round_scale=True) == "mxfp8"
    assert OV.check_flags(True, True, False, True, False) == "mxfp8"
    with pytest.raises(ep.EpError):
        ep.quant_mode(use_fp8=True, round_scale=True)
    with pytest.raises(ValueError):
        OV.check_flags(True, False, False, True, False)
    for flags in [dict(use_fp8=False), dict(use_fp8=True), dict(use_fp8=True, use_ue8m0=True),
                  dict(use_fp8=True, use_mxfp4=True)]:
        assert ep.quant_mode(**flags) == OV.check_flags(flags.get("use_fp8"), flags.get("use_ue8m0", False),
                                                        flags.get("use_mxfp4", False), False, False)


def test_moe_packed_bytes(ep):
    assert ep.ep_moe_packed_bytes(6, 6144, 7168) == (6 * 6144 * 7168, 6 * (6144 // 32) * 28 * 256)
    assert ep.ep_moe_packed_bytes(1, 32, 320) == (32 * 320, 2 * 256)          # 5 steps -> 2 spans
    for bad in ((0, 32, 64), (1, 48, 64), (1, 32, 96), (513, 32, 64)):
        with pytest.raises(ep.EpError):
            ep.ep_moe_packed_bytes(*bad)


MOE_BAD = [(dict(hidden=96), 1), (dict(hidden=192), 1), (dict(inter=100), 1), (dict(out_quant=2), 1), (dict(x=None), 1),
           (dict(w1=FAKE + 8), 1), (dict(out_bytes=10), 3)]


@pytest.mark.parametrize("kw,code", MOE_BAD)
def test_moe_gmm1_rejects(ep, kw, code):
    h = _handle(ep)
    rc = ep._lib.ep_moe_gmm1(ctypes.byref(h), None, kw.get("x", FAKE), 1 << 30, kw.get("hidden", 256),
                             kw.get("inter", 128), kw.get("w1", FAKE), FAKE, kw.get("out_quant", 3), FAKE,
                             kw.get("out_bytes", 1 << 30), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_moe_gmm1")


def test_moe_gmm2_rejects(ep):
    h = _handle(ep)
    assert ep._lib.ep_moe_gmm2(ctypes.byref(h), None, FAKE, 1 << 30, 128, 192, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert ep._lib.ep_moe_gmm2(ctypes.byref(h), None, FAKE, 1 << 30, 96, 256, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert ep._lib.ep_moe_gmm2(ctypes.byref(h), None, FAKE, 1 << 30, 192, 256, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert ep._lib.ep_moe_gmm2(ctypes.byref(h), None, FAKE, 8, 128, 256, FAKE, FAKE, FAKE, 1 << 30, None) == 3


def test_noalloc_refuses_a_layout_beyond_its_static_workspace(ep):
    """ep_layout_dispatch_noalloc: num_max_dispatch_tokens * k = 2^20 pairs
    needs over 8 MiB of workspace, more than the library's static 4 MiB; the
    call returns EP_ERR_BUFFER_TOO_SMALL before touching the device."""
    tmax, k, E = 1 << 17, 8, 256
    assert ep.ep_workspace_bytes(tmax, k, E) > ep.STATIC_WORKSPACE_BYTES
    h = ep.ep_handle_t()
    rc = ep._lib.ep_layout_dispatch_noalloc(FAKE, 1, 16, k, tmax, E, 1, 0, FAKE, None, FAKE, 7168, None, 3, FAKE,
                                            1 << 40, None, ctypes.byref(h), None)
    assert rc == ep.EP_ERR_BUFFER_TOO_SMALL
    assert ep.ep_last_error().startswith("ep_layout_dispatch_noalloc") and "static" in ep.ep_last_error()
