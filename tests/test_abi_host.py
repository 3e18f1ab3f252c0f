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
    assert ep.ep_abi_version() == 1


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


def _handle(ep, T=4, k=2, tmax=8, E=8):
    h = ep.ep_handle_t()
    h.num_tokens, h.num_max_tokens, h.max_rows = T, tmax, tmax * k
    h.num_topk, h.num_experts = k, E
    h.offsets = h.slot = h.row_src = h.status = FAKE
    return h


DISPATCH_BAD = [
    (dict(hidden=0), 1), (dict(hidden=48), 1), (dict(hidden=96, quant=2), 1), (dict(quant=7), 1),
    (dict(hidden=65568), 2), (dict(x=None), 1), (dict(x=FAKE + 8), 1), (dict(recv=None), 1),
    (dict(recv=FAKE + 8), 1), (dict(recv_bytes=10), 3), (dict(rw=FAKE, w=None), 1), (dict(w=FAKE + 2), 1),
    (dict(h_bad="k"), 1), (dict(h_bad="rows"), 1), (dict(h_bad="ptr"), 1), (dict(h_none=True), 1),
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
    hp = None if kw.get("h_none") else ctypes.byref(h)
    hidden = kw.get("hidden", 256)
    quant = kw.get("quant", 3)
    rc = ep._lib.ep_dispatch(hp, kw.get("x", FAKE), hidden, kw.get("w", None), quant, kw.get("recv", FAKE),
                             kw.get("recv_bytes", 1 << 30), kw.get("rw", None), None)
    assert rc == code, ep.ep_last_error()
    assert ep.ep_last_error().startswith("ep_dispatch")


COMBINE_BAD = [
    (dict(hidden=40), 1), (dict(quant=-1), 1), (dict(inp=None), 1), (dict(inp=FAKE + 4), 1),
    (dict(in_bytes=5), 3), (dict(w=None), 1), (dict(out=None), 1), (dict(out=FAKE + 2), 1),
    (dict(hidden=128 + 32, quant=2), 1),
]


@pytest.mark.parametrize("kw,code", COMBINE_BAD)
def test_combine_rejects(ep, kw, code):
    h = _handle(ep)
    rc = ep._lib.ep_combine(ctypes.byref(h), kw.get("inp", FAKE), kw.get("in_bytes", 1 << 30),
                            kw.get("quant", 0), kw.get("hidden", 256), kw.get("w", FAKE), kw.get("out", FAKE),
                            None)
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
                                         (96, "mxfp8"), (7168, "mxfp4"), (1024, "mxfp4")])
@pytest.mark.parametrize("rows", [0, 1, 37, 131072])
def test_buffer_bytes_matches_oracle(ep, hidden, mode, rows):
    assert ep.ep_buffer_bytes(rows, hidden, mode) == OD.buffer_bytes(rows, hidden, mode)


def test_buffer_bytes_rejects(ep):
    with pytest.raises(ep.EpError) as e:
        ep.ep_buffer_bytes(10, 100, "none")
    assert e.value.code == 1
    with pytest.raises(ep.EpError):
        ep.ep_buffer_bytes(-1, 128, "none")
    with pytest.raises(ep.EpError):
        ep.ep_buffer_bytes(1, 96, "fp8_b128")


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
    for flags in [dict(use_fp8=False), dict(use_fp8=True), dict(use_fp8=True, use_ue8m0=True),
                  dict(use_fp8=True, use_mxfp4=True)]:
        assert ep.quant_mode(**flags) == OV.check_flags(flags.get("use_fp8"), flags.get("use_ue8m0", False),
                                                        flags.get("use_mxfp4", False), False, False)
