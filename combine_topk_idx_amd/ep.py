"""ctypes binding of libep.so (argument marshalling only).

The functions ``ep_workspace_bytes``, ``ep_workspace_bytes_ex``,
``ep_layout_rows``, ``ep_buffer_bytes``, ``ep_layout``, ``ep_layout_ex``,
``ep_dispatch``, ``ep_layout_dispatch``, ``ep_layout_dispatch_noalloc``,
``ep_combine``, ``ep_combine_backward``,
``ep_moe_packed_bytes``, ``ep_moe_pack_weights``, ``ep_moe_gmm1``,
``ep_moe_gmm2``, ``ep_read_status``,
``ep_last_error`` and ``ep_abi_version`` have the names and arguments of the C ABI in
``include/ep.h``; torch tensors stand in for device pointers and torch's
current stream is used unless one is passed.  Every computation runs in the
library's HIP kernels.  Importing this module loads the library and raises
``ImportError`` if it is missing: there is no fallback.

``low_latency_dispatch`` / ``low_latency_combine`` follow the argument lists of
the "Low-Latency Mode API" page: they allocate the outputs with torch and call
the same entry points.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m combine_topk_idx_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_BUFFER_TOO_SMALL, EP_ERR_HIP = range(5)
EP_IDX_INT32, EP_IDX_INT64 = 0, 1
QUANT = {"none": 0, "int8_token": 1, "fp8_b128": 2, "mxfp8": 3, "mxfp4": 4, "fp8_b128_pow2": 5,
         "fp8_b128_ue8m0": 6}
EP_RECV_INTERLEAVED = 0x100
EP_STATUS_ID_OUT_OF_RANGE = 1
EP_STATUS_CAPACITY_OVERFLOW = 2
EP_STATUS_COMBINE_MISMATCH = 4

SYMBOLS = ("ep_workspace_bytes", "ep_workspace_bytes_ex", "ep_layout_rows", "ep_buffer_bytes", "ep_layout",
           "ep_layout_ex", "ep_dispatch", "ep_layout_dispatch", "ep_layout_dispatch_noalloc", "ep_combine",
           "ep_combine_backward", "ep_moe_packed_bytes", "ep_moe_pack_weights", "ep_moe_gmm1", "ep_moe_gmm2",
           "ep_read_status", "ep_last_error", "ep_abi_version")
STATIC_WORKSPACE_BYTES = 4 << 20   # the static workspace of ep_layout_dispatch_noalloc


class ep_handle_t(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("num_max_tokens", ctypes.c_int64),
        ("max_rows", ctypes.c_int64),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("row_align", ctypes.c_int32),
        ("expert_capacity", ctypes.c_int32),
        ("offsets", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("row_src", ctypes.c_void_p),
        ("status", ctypes.c_void_p),
    ]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_lib.ep_workspace_bytes.argtypes = [_i64, _i32, _i32]
_lib.ep_workspace_bytes.restype = _sz
_lib.ep_workspace_bytes_ex.argtypes = [_i64, _i32, _i32, _i32, _i32]
_lib.ep_workspace_bytes_ex.restype = _sz
_lib.ep_layout_rows.argtypes = [_i64, _i32, _i32, _i32, _i32]
_lib.ep_layout_rows.restype = _i64
_lib.ep_buffer_bytes.argtypes = [_i64, _i32, ctypes.c_int, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
_lib.ep_buffer_bytes.restype = ctypes.c_int
_lib.ep_layout.argtypes = [_vp, ctypes.c_int, _i64, _i32, _i64, _i32, _vp, _vp, _vp, _sz,
                           ctypes.POINTER(ep_handle_t), _vp]
_lib.ep_layout.restype = ctypes.c_int
_lib.ep_layout_ex.argtypes = [_vp, ctypes.c_int, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                              ctypes.POINTER(ep_handle_t), _vp]
_lib.ep_layout_ex.restype = ctypes.c_int
_lib.ep_dispatch.argtypes = [ctypes.POINTER(ep_handle_t), _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp, _vp]
_lib.ep_dispatch.restype = ctypes.c_int
_lib.ep_layout_dispatch.argtypes = [_vp, ctypes.c_int, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                    _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp, ctypes.POINTER(ep_handle_t), _vp]
_lib.ep_layout_dispatch.restype = ctypes.c_int
_lib.ep_layout_dispatch_noalloc.argtypes = [_vp, ctypes.c_int, _i64, _i32, _i64, _i32, _i32, _i32, _vp, _vp,
                                            _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp, ctypes.POINTER(ep_handle_t),
                                            _vp]
_lib.ep_layout_dispatch_noalloc.restype = ctypes.c_int
_lib.ep_combine.argtypes = [ctypes.POINTER(ep_handle_t), _vp, _sz, ctypes.c_int, _i32, _vp, ctypes.c_int, _vp, _vp,
                            _vp]
_lib.ep_combine.restype = ctypes.c_int
_lib.ep_combine_backward.argtypes = [ctypes.POINTER(ep_handle_t), _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp]
_lib.ep_combine_backward.restype = ctypes.c_int
_lib.ep_moe_packed_bytes.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
_lib.ep_moe_packed_bytes.restype = ctypes.c_int
_lib.ep_moe_pack_weights.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
_lib.ep_moe_pack_weights.restype = ctypes.c_int
_lib.ep_moe_gmm1.argtypes = [ctypes.POINTER(ep_handle_t), _vp, _vp, _sz, _i32, _i32, _vp, _vp, ctypes.c_int, _vp,
                             _sz, _vp]
_lib.ep_moe_gmm1.restype = ctypes.c_int
_lib.ep_moe_gmm2.argtypes = [ctypes.POINTER(ep_handle_t), _vp, _vp, _sz, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.ep_moe_gmm2.restype = ctypes.c_int
_lib.ep_read_status.argtypes = [ctypes.POINTER(ep_handle_t), ctypes.POINTER(ctypes.c_uint32), _vp]
_lib.ep_read_status.restype = ctypes.c_int
_lib.ep_last_error.argtypes = []
_lib.ep_last_error.restype = ctypes.c_char_p
_lib.ep_abi_version.argtypes = []
_lib.ep_abi_version.restype = _i32


class EpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _check(code: int) -> None:
    if code != EP_OK:
        raise EpError(code, ep_last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


try:
    _raw_stream = torch._C._cuda_getCurrentRawStream   # int handle, no Stream object
except AttributeError:  # pragma: no cover
    _raw_stream = None


def _stream(stream) -> Optional[int]:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _quant(q, interleaved: bool = False) -> int:
    v = QUANT[q] if isinstance(q, str) else int(q)
    return v | EP_RECV_INTERLEAVED if interleaved else v


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_args(*specs) -> None:
    """Host checks of tensor arguments before their pointers reach the
    library, which can only check pointers and byte counts.  Each spec is
    (tensor, name, dtype, shape, min_numel) with None for "any"; raw integer
    pointers and None tensors pass unchecked.  Every tensor's dtype, shape,
    density and size, then that all of them are on one GPU.  The common case
    (everything valid) reads each attribute once; the messages are built
    only on failure."""
    dev, dev_name = -2, None
    for t, name, dtype, shape, min_numel in specs:
        if t is None or type(t) is int:
            continue
        if not isinstance(t, torch.Tensor):
            raise EpError(EP_ERR_INVALID_ARG, f"{name} must be a tensor")
        if not ((dtype is None or t.dtype is dtype) and (shape is None or t.shape == shape) and t.is_contiguous()
                and (min_numel is None or t.numel() >= min_numel)):
            _explain(t, name, dtype, shape, min_numel)
        d = t.get_device()
        if dev == -2:
            dev, dev_name = d, name
        elif d != dev:
            raise EpError(EP_ERR_INVALID_ARG, f"{name} is on {t.device}, {dev_name} on another device")
    if dev == -1:
        raise EpError(EP_ERR_INVALID_ARG, f"{dev_name} must be a GPU tensor (got cpu)")


def _explain(t, name, dtype, shape, min_numel) -> None:
    """Raises the error for a tensor that failed the checks of _check_args."""
    if dtype is not None and t.dtype != dtype:
        raise EpError(EP_ERR_INVALID_ARG, f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise EpError(EP_ERR_INVALID_ARG, f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise EpError(EP_ERR_INVALID_ARG, f"{name} must be contiguous")
    raise EpError(EP_ERR_INVALID_ARG, f"{name} holds {t.numel()} elements, needs {min_numel}")


# ---------------------------------------------------------------------------
# C ABI, one function each
# ---------------------------------------------------------------------------


def ep_abi_version() -> int:
    return _lib.ep_abi_version()


def ep_last_error() -> str:
    return (_lib.ep_last_error() or b"").decode()


def ep_workspace_bytes(num_max_dispatch_tokens: int, num_topk: int, num_experts: int) -> int:
    return _lib.ep_workspace_bytes(num_max_dispatch_tokens, num_topk, num_experts)


def ep_workspace_bytes_ex(num_max_dispatch_tokens: int, num_topk: int, num_experts: int, row_align: int = 1,
                          expert_capacity: int = 0) -> int:
    return _lib.ep_workspace_bytes_ex(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity)


def ep_layout_rows(num_max_dispatch_tokens: int, num_topk: int, num_experts: int, row_align: int = 1,
                   expert_capacity: int = 0) -> int:
    return _lib.ep_layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity)


def ep_buffer_bytes(rows: int, hidden: int, quant, interleaved: bool = False) -> tuple[int, int]:
    """(total bytes, scale offset): the scale region's start, or for
    interleaved rows the scales' offset inside a row."""
    total, off = _sz(0), _sz(0)
    _check(_lib.ep_buffer_bytes(rows, hidden, _quant(quant, interleaved), ctypes.byref(total), ctypes.byref(off)))
    return total.value, off.value


def _idx_args(topk_idx, num_tokens, num_topk, idx_dtype):
    if isinstance(topk_idx, torch.Tensor):
        if topk_idx.dim() != 2 or not topk_idx.is_contiguous():
            raise EpError(EP_ERR_INVALID_ARG, "topk_idx must be a contiguous [num_tokens, num_topk] tensor")
        if topk_idx.dtype not in (torch.int32, torch.int64):
            raise EpError(EP_ERR_INVALID_ARG, "topk_idx dtype must be int32 or int64")
        num_tokens, num_topk = topk_idx.shape
        idx_dtype = EP_IDX_INT64 if topk_idx.dtype == torch.int64 else EP_IDX_INT32
    return num_tokens, num_topk, idx_dtype


def _layout_specs(topk_idx, num_experts, recv_count, workspace, cum) -> list:
    return [(topk_idx, "topk_idx", None, None, None),
            (recv_count, "recv_count", torch.int64, None, num_experts),
            (workspace, "workspace", None, None, None),
            (cum, "cumulative_recv_stats", torch.int32, None, num_experts)]


def ep_layout(topk_idx, num_experts: int, num_max_dispatch_tokens: int, recv_count, workspace,
              cumulative_recv_stats=None, *, num_tokens=None, num_topk=None, idx_dtype=None,
              stream=None) -> ep_handle_t:
    """topk_idx: device tensor [T, k] int32/int64 (or a raw pointer with
    num_tokens / num_topk / idx_dtype given).  Returns the handle."""
    num_tokens, num_topk, idx_dtype = _idx_args(topk_idx, num_tokens, num_topk, idx_dtype)
    _check_args(*_layout_specs(topk_idx, num_experts, recv_count, workspace, cumulative_recv_stats))
    h = ep_handle_t()
    _check(_lib.ep_layout(_ptr(topk_idx), idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                          num_experts, _ptr(recv_count), _ptr(cumulative_recv_stats), _ptr(workspace),
                          _nbytes(workspace) if isinstance(workspace, torch.Tensor) else 0,
                          ctypes.byref(h), _stream(stream)))
    return h


def ep_layout_ex(topk_idx, num_experts: int, num_max_dispatch_tokens: int, row_align: int, expert_capacity: int,
                 recv_count, workspace, cumulative_recv_stats=None, *, num_tokens=None, num_topk=None,
                 idx_dtype=None, stream=None) -> ep_handle_t:
    """As ep_layout, with aligned (row_align) or capacity-padded
    (expert_capacity) expert blocks."""
    num_tokens, num_topk, idx_dtype = _idx_args(topk_idx, num_tokens, num_topk, idx_dtype)
    _check_args(*_layout_specs(topk_idx, num_experts, recv_count, workspace, cumulative_recv_stats))
    h = ep_handle_t()
    _check(_lib.ep_layout_ex(_ptr(topk_idx), idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                             num_experts, row_align, expert_capacity, _ptr(recv_count),
                             _ptr(cumulative_recv_stats), _ptr(workspace),
                             _nbytes(workspace) if isinstance(workspace, torch.Tensor) else 0,
                             ctypes.byref(h), _stream(stream)))
    return h


def _dispatch_specs(T: int, k: int, max_rows: int, x, hidden: int, recv_buf, topk_weights, recv_weights) -> list:
    return [(x, "x", torch.bfloat16, (T, hidden), None),
            (recv_buf, "recv_buf", None, None, None),
            (topk_weights, "topk_weights", torch.float32, (T, k), None),
            (recv_weights, "recv_weights", torch.float32, None, max_rows)]


def ep_dispatch(handle: ep_handle_t, x, hidden: int, quant, recv_buf, topk_weights=None,
                recv_weights=None, *, recv_buf_bytes=None, interleaved=False, stream=None) -> None:
    _check_args(*_dispatch_specs(handle.num_tokens, handle.num_topk, handle.max_rows, x, hidden, recv_buf,
                                 topk_weights, recv_weights))
    nbytes = _nbytes(recv_buf) if recv_buf_bytes is None else recv_buf_bytes
    _check(_lib.ep_dispatch(ctypes.byref(handle), _ptr(x), hidden, _ptr(topk_weights), _quant(quant, interleaved),
                            _ptr(recv_buf), nbytes, _ptr(recv_weights), _stream(stream)))


def ep_layout_dispatch(topk_idx, num_experts: int, num_max_dispatch_tokens: int, recv_count, workspace,
                       x, hidden: int, quant, recv_buf, topk_weights=None, recv_weights=None,
                       cumulative_recv_stats=None, *, row_align: int = 1, expert_capacity: int = 0,
                       num_tokens=None, num_topk=None, idx_dtype=None, recv_buf_bytes=None, interleaved=False,
                       stream=None) -> ep_handle_t:
    """ep_layout_ex and ep_dispatch in one call (one launch for compact
    layouts and capacity blocks of at most 2048 pairs).  Returns the handle."""
    num_tokens, num_topk, idx_dtype = _idx_args(topk_idx, num_tokens, num_topk, idx_dtype)
    rows = max(ep_layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity), 0)
    _check_args(*_layout_specs(topk_idx, num_experts, recv_count, workspace, cumulative_recv_stats),
                *_dispatch_specs(num_tokens, num_topk, rows, x, hidden, recv_buf, topk_weights, recv_weights))
    nbytes = _nbytes(recv_buf) if recv_buf_bytes is None else recv_buf_bytes
    h = ep_handle_t()
    _check(_lib.ep_layout_dispatch(_ptr(topk_idx), idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                                   num_experts, row_align, expert_capacity, _ptr(recv_count),
                                   _ptr(cumulative_recv_stats), _ptr(workspace),
                                   _nbytes(workspace) if isinstance(workspace, torch.Tensor) else 0,
                                   _ptr(x), hidden, _ptr(topk_weights), _quant(quant, interleaved), _ptr(recv_buf),
                                   nbytes, _ptr(recv_weights), ctypes.byref(h), _stream(stream)))
    return h


def ep_layout_dispatch_noalloc(topk_idx, num_experts: int, num_max_dispatch_tokens: int, recv_count, x,
                               hidden: int, quant, recv_buf, topk_weights=None, recv_weights=None,
                               cumulative_recv_stats=None, *, row_align: int = 1, expert_capacity: int = 0,
                               num_tokens=None, num_topk=None, idx_dtype=None, recv_buf_bytes=None,
                               interleaved=False, stream=None) -> ep_handle_t:
    """ep_layout_dispatch with the library's static workspace (no workspace
    argument, nothing allocated).  The handle is valid until the next call of
    this function on the same device."""
    num_tokens, num_topk, idx_dtype = _idx_args(topk_idx, num_tokens, num_topk, idx_dtype)
    rows = max(ep_layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity), 0)
    _check_args(*_layout_specs(topk_idx, num_experts, recv_count, None, cumulative_recv_stats),
                *_dispatch_specs(num_tokens, num_topk, rows, x, hidden, recv_buf, topk_weights, recv_weights))
    nbytes = _nbytes(recv_buf) if recv_buf_bytes is None else recv_buf_bytes
    h = ep_handle_t()
    _check(_lib.ep_layout_dispatch_noalloc(_ptr(topk_idx), idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                                           num_experts, row_align, expert_capacity, _ptr(recv_count),
                                           _ptr(cumulative_recv_stats), _ptr(x), hidden, _ptr(topk_weights),
                                           _quant(quant, interleaved), _ptr(recv_buf), nbytes, _ptr(recv_weights),
                                           ctypes.byref(h), _stream(stream)))
    return h


def ep_combine(handle: ep_handle_t, expert_out, in_quant, hidden: int, topk_idx, topk_weights, out, *,
               idx_dtype=None, expert_out_bytes=None, interleaved=False, stream=None) -> None:
    """topk_idx: the [T, k] ids given to the layout (a device tensor, or a
    raw pointer with idx_dtype); a mismatch with the handle sets
    EP_STATUS_COMBINE_MISMATCH."""
    T, k = handle.num_tokens, handle.num_topk
    if isinstance(topk_idx, torch.Tensor):
        if topk_idx.dtype is torch.int64:
            idx_dtype = EP_IDX_INT64
        elif topk_idx.dtype is torch.int32:
            idx_dtype = EP_IDX_INT32
        else:
            raise EpError(EP_ERR_INVALID_ARG, "topk_idx dtype must be int32 or int64")
    elif idx_dtype is None:
        raise EpError(EP_ERR_INVALID_ARG, "idx_dtype is required with a raw topk_idx pointer")
    _check_args((expert_out, "expert_out", None, None, None), (topk_idx, "topk_idx", None, (T, k), None),
                (topk_weights, "topk_weights", torch.float32, (T, k), None),
                (out, "out", torch.bfloat16, (T, hidden), None))
    nbytes = _nbytes(expert_out) if expert_out_bytes is None else expert_out_bytes
    _check(_lib.ep_combine(ctypes.byref(handle), _ptr(expert_out), nbytes, _quant(in_quant, interleaved), hidden,
                           _ptr(topk_idx), idx_dtype, _ptr(topk_weights), _ptr(out), _stream(stream)))


def ep_combine_backward(handle: ep_handle_t, grad_out, hidden: int, quant, grad_buf, topk_weights=None, *,
                        grad_buf_bytes=None, interleaved=False, stream=None) -> None:
    _check_args((grad_out, "grad_out", torch.bfloat16, (handle.num_tokens, hidden), None),
                (grad_buf, "grad_buf", None, None, None),
                (topk_weights, "topk_weights", torch.float32, (handle.num_tokens, handle.num_topk), None))
    nbytes = _nbytes(grad_buf) if grad_buf_bytes is None else grad_buf_bytes
    _check(_lib.ep_combine_backward(ctypes.byref(handle), _ptr(grad_out), hidden, _ptr(topk_weights),
                                    _quant(quant, interleaved), _ptr(grad_buf), nbytes, _stream(stream)))


def ep_moe_packed_bytes(num_experts: int, rows: int, k: int) -> tuple[int, int]:
    c, sc = _sz(0), _sz(0)
    _check(_lib.ep_moe_packed_bytes(num_experts, rows, k, ctypes.byref(c), ctypes.byref(sc)))
    return c.value, sc.value


def ep_moe_pack_weights(codes, scales, num_experts: int, rows: int, k: int, gate_up: bool, packed_codes,
                        packed_scales, *, stream=None) -> None:
    _check(_lib.ep_moe_pack_weights(_ptr(codes), _ptr(scales), num_experts, rows, k, int(gate_up), _ptr(packed_codes),
                                    _ptr(packed_scales), _stream(stream)))


def pack_moe_weights(codes, scales, gate_up: bool, *, stream=None):
    """Device tensors codes [E, N, K] uint8 and scales [E, N, K/32] uint8 ->
    (packed codes, packed scales) uint8 device tensors."""
    E, N, K = codes.shape
    cb, sb = ep_moe_packed_bytes(E, N, K)
    pc = torch.empty(cb, dtype=torch.uint8, device=codes.device)
    ps = torch.empty(sb, dtype=torch.uint8, device=codes.device)
    ep_moe_pack_weights(codes, scales, E, N, K, gate_up, pc, ps, stream=stream)
    return pc, ps


def _check_moe_args(handle: ep_handle_t, recv_count, weights, **bufs) -> None:
    """weights: (codes, scales, rows, k, names) of packed weights, which must be
    the 1-D uint8 tensors ep_moe_pack_weights fills for exactly the handle's
    num_experts experts (the packing is step-major, so weights packed for
    another expert count would be read at the wrong places).  Shapes the
    library rejects anyway are left to its own message."""
    codes, scales, rows, k, (cn, sn) = weights
    try:
        cb, sb = ep_moe_packed_bytes(handle.num_experts, rows, k)
    except EpError:
        cb = sb = None
    _check_args((codes, cn, torch.uint8, None if cb is None else (cb,), None),
                (scales, sn, torch.uint8, None if sb is None else (sb,), None),
                *[(b, n, None, None, None) for n, b in bufs.items()],
                (recv_count, "recv_count", torch.int64, None, handle.num_experts))


def ep_moe_gmm1(handle: ep_handle_t, x_buf, hidden: int, inter: int, w1, w1_scales, out_quant, out_buf, *,
                recv_count=None, x_buf_bytes=None, out_buf_bytes=None, stream=None) -> None:
    _check_moe_args(handle, recv_count, (w1, w1_scales, 2 * inter, hidden, ("w1", "w1_scales")), x_buf=x_buf,
                    out_buf=out_buf)
    _check(_lib.ep_moe_gmm1(ctypes.byref(handle), _ptr(recv_count), _ptr(x_buf),
                            _nbytes(x_buf) if x_buf_bytes is None else x_buf_bytes, hidden, inter, _ptr(w1),
                            _ptr(w1_scales), _quant(out_quant), _ptr(out_buf),
                            _nbytes(out_buf) if out_buf_bytes is None else out_buf_bytes, _stream(stream)))


def ep_moe_gmm2(handle: ep_handle_t, a_buf, inter: int, hidden: int, w2, w2_scales, out_buf, *,
                recv_count=None, a_buf_bytes=None, out_buf_bytes=None, stream=None) -> None:
    _check_moe_args(handle, recv_count, (w2, w2_scales, hidden, inter, ("w2", "w2_scales")), a_buf=a_buf,
                    out_buf=out_buf)
    _check(_lib.ep_moe_gmm2(ctypes.byref(handle), _ptr(recv_count), _ptr(a_buf),
                            _nbytes(a_buf) if a_buf_bytes is None else a_buf_bytes, inter, hidden, _ptr(w2),
                            _ptr(w2_scales), _ptr(out_buf), _nbytes(out_buf) if out_buf_bytes is None else out_buf_bytes,
                            _stream(stream)))


def ep_read_status(handle: ep_handle_t, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(_lib.ep_read_status(ctypes.byref(handle), ctypes.byref(flags), _stream(stream)))
    return flags.value


# ---------------------------------------------------------------------------
# "Low-Latency Mode API"-shaped wrappers
# ---------------------------------------------------------------------------


@dataclass
class Handle:
    """What low_latency_dispatch hands to low_latency_combine: the C handle
    plus the tensors its pointers live in (kept alive here)."""
    c: ep_handle_t
    workspace: torch.Tensor
    hidden: int
    quant: str
    topk_idx_shape: tuple
    topk_idx_dtype: torch.dtype


def quant_mode(use_fp8=True, use_ue8m0=False, use_mxfp4=False, quant=None, round_scale=False) -> str:
    """Flag mapping of the "Low-Latency Mode API" page: no use_fp8 -> bf16;
    use_fp8 -> int8 per token; + use_ue8m0 -> MXFP8; + use_mxfp4 -> MXFP4;
    round_scale goes with use_ue8m0 (whose scales are powers of two
    already).  ``quant=`` names a mode directly, e.g. "fp8_b128" (e4m3 with
    per-128-channel scales) or its power-of-two variants "fp8_b128_pow2" /
    "fp8_b128_ue8m0"."""
    if quant is not None:
        if quant not in QUANT:
            raise EpError(EP_ERR_INVALID_ARG, f"unknown quant {quant!r}")
        return quant
    if round_scale and not use_ue8m0:
        raise EpError(EP_ERR_INVALID_ARG, "round_scale is used together with use_ue8m0")
    if (use_ue8m0 or use_mxfp4) and not use_fp8:
        raise EpError(EP_ERR_INVALID_ARG, "use_ue8m0 / use_mxfp4 require use_fp8")
    if use_ue8m0 and use_mxfp4:
        raise EpError(EP_ERR_INVALID_ARG, "use_ue8m0 and use_mxfp4 are exclusive")
    if not use_fp8:
        return "none"
    return "mxfp4" if use_mxfp4 else ("mxfp8" if use_ue8m0 else "int8_token")


def split_recv(buf: torch.Tensor, rows: int, hidden: int, quant: str):
    """Views of a receive buffer in the shapes of the page's Return Values."""
    total, off = ep_buffer_bytes(rows, hidden, quant)
    q = quant
    if q == "none":
        return buf[: rows * hidden * 2].view(torch.bfloat16).view(rows, hidden)
    if q == "int8_token":
        return (buf[: rows * hidden].view(torch.int8).view(rows, hidden),
                buf[off: off + rows * 4].view(torch.float32))
    if q in ("fp8_b128", "fp8_b128_pow2"):
        return (buf[: rows * hidden].view(torch.float8_e4m3fn).view(rows, hidden),
                buf[off: off + rows * (hidden // 128) * 4].view(torch.float32).view(rows, hidden // 128))
    if q == "fp8_b128_ue8m0":
        return (buf[: rows * hidden].view(torch.float8_e4m3fn).view(rows, hidden),
                buf[off: off + rows * (hidden // 128)].view(torch.float8_e8m0fnu).view(rows, hidden // 128))
    if q == "mxfp8":
        return (buf[: rows * hidden].view(torch.float8_e4m3fn).view(rows, hidden),
                buf[off: off + rows * (hidden // 32)].view(torch.float8_e8m0fnu))
    return (buf[: rows * hidden // 2].view(torch.float4_e2m1fn_x2).view(rows, hidden // 2),
            buf[off: off + rows * (hidden // 32)].view(torch.float8_e8m0fnu))


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_max_dispatch_tokens_per_rank: int,
                         num_experts: int, cumulative_local_expert_recv_stats=None, use_fp8: bool = True,
                         round_scale: bool = False, use_ue8m0: bool = False, use_mxfp4: bool = False,
                         async_finish: bool = False, return_recv_hook: bool = False, topk_weights=None,
                         quant: Optional[str] = None, row_align: int = 1, expert_capacity: int = 0):
    """Returns (recv_x, recv_count, handle, event, hook) with event and hook
    None (there is no transport to overlap or to wait for).  ``row_align`` /
    ``expert_capacity`` select aligned or capacity-padded expert blocks; with
    a capacity C the data views are shaped [num_experts, C, ...]."""
    if return_recv_hook:
        raise EpError(EP_ERR_UNSUPPORTED, "return_recv_hook is not supported")
    q = quant_mode(use_fp8, use_ue8m0, use_mxfp4, quant, round_scale)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise EpError(EP_ERR_INVALID_ARG, "x must be a contiguous bf16 [num_tokens, hidden] tensor")
    T, H = x.shape
    if topk_idx.dim() != 2 or topk_idx.shape[0] != T:
        raise EpError(EP_ERR_INVALID_ARG, "topk_idx must be [num_tokens, num_topk]")
    k = topk_idx.shape[1]
    dev = x.device
    _check_args((x, "x", None, None, None), (topk_idx, "topk_idx", None, None, None),
                (topk_weights, "topk_weights", torch.float32, (T, k), None))
    ws = torch.empty(max(ep_workspace_bytes_ex(num_max_dispatch_tokens_per_rank, k, num_experts, row_align,
                                               expert_capacity), 1), dtype=torch.uint8, device=dev)
    recv_count = torch.empty(num_experts, dtype=torch.int64, device=dev)
    rows = ep_layout_rows(num_max_dispatch_tokens_per_rank, k, num_experts, row_align, expert_capacity)
    if rows < 0:
        raise EpError(EP_ERR_INVALID_ARG, "receive rows out of range")
    total, _ = ep_buffer_bytes(rows, H, q)
    buf = torch.empty(max(total, 16), dtype=torch.uint8, device=dev)
    recv_w = None
    if topk_weights is not None:
        recv_w = torch.empty(max(rows, 1), dtype=torch.float32, device=dev)
    h = ep_layout_dispatch(topk_idx, num_experts, num_max_dispatch_tokens_per_rank, recv_count, ws, x, H, q, buf,
                           topk_weights, recv_w, cumulative_local_expert_recv_stats, row_align=row_align,
                           expert_capacity=expert_capacity)
    handle = Handle(h, ws, H, q, tuple(topk_idx.shape), topk_idx.dtype)
    recv_x = split_recv(buf, rows, H, q)
    if expert_capacity > 0:
        if isinstance(recv_x, tuple):
            recv_x = (recv_x[0].view(num_experts, expert_capacity, -1),) + recv_x[1:]
        else:
            recv_x = recv_x.view(num_experts, expert_capacity, H)
    if recv_w is not None:
        handle.recv_weights = recv_w
    return recv_x, recv_count, handle, None, None


def low_latency_combine(x, topk_idx: torch.Tensor, topk_weights: torch.Tensor, handle: Handle,
                        zero_copy: bool = False, async_finish: bool = False, return_recv_hook: bool = False,
                        out: Optional[torch.Tensor] = None, in_quant: str = "none"):
    """x: bf16 [max_rows, hidden] expert outputs ([num_experts, C, hidden]
    for a capacity-padded layout), or a raw uint8 receive-format buffer with
    ``in_quant``.  Returns (combined_x, event, hook)."""
    if zero_copy or return_recv_hook:
        raise EpError(EP_ERR_UNSUPPORTED, "zero_copy / return_recv_hook are not supported")
    if tuple(topk_idx.shape) != handle.topk_idx_shape or topk_idx.dtype != handle.topk_idx_dtype:
        raise EpError(EP_ERR_INVALID_ARG, "topk_idx does not match the one given to dispatch")
    T, H = handle.topk_idx_shape[0], handle.hidden
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=handle.workspace.device)
    ep_combine(handle.c, x, in_quant, H, topk_idx, topk_weights, out)
    return out, None, None
