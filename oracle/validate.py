"""Argument rules of the oracle (test infrastructure only).

The C ABI checks its arguments on the host before any launch and returns an
error code ("DeepEP topk_idx_t Custom Dtype Requirements", "Runtime
Validation": checks halt before any GPU work; "Tensor Requirements and
Constraints": exact index dtype, two dimensions [num_tokens, num_topk],
contiguous).  The numeric limits follow "Low-Latency Mode API",
Constraints: num_topk in (0, 16], num_experts in (0, 512], hidden a positive
multiple of 32, and the token count bounded by num_max_dispatch_tokens_per_rank
(read as "at most": the page gives a strict and a non-strict bound in two
places).  The per-128 FP8 mode also needs
hidden % 128 == 0 (its blocks are 128 wide).

``check_*`` raise ``ValueError`` exactly where the ABI returns
``EP_ERR_INVALID_ARG`` and ``NotImplementedError`` where it returns
``EP_ERR_UNSUPPORTED``.  Parity: pinned case by case against the ABI's
return codes in ``tests/test_abi_host.py`` (the rules are the pages' own
list, so the cases themselves are the pin).
"""

from __future__ import annotations

MAX_TOPK = 16
MAX_EXPERTS = 512
QUANT_MODES = ("none", "int8_token", "fp8_b128", "mxfp8", "mxfp4", "fp8_b128_pow2", "fp8_b128_ue8m0")


def check_layout(num_tokens: int, num_topk: int, num_max_dispatch_tokens: int, num_experts: int) -> None:
    if not (0 < num_topk <= MAX_TOPK):
        raise ValueError("num_topk must be in (0, 16]")
    if not (0 < num_experts <= MAX_EXPERTS):
        raise ValueError("num_experts must be in (0, 512]")
    if num_tokens < 0 or num_max_dispatch_tokens < 0:
        raise ValueError("negative token count")
    if num_tokens > num_max_dispatch_tokens:
        raise ValueError("num_tokens exceeds num_max_dispatch_tokens")
    if num_max_dispatch_tokens * num_topk > 2 ** 31 - 1:
        raise ValueError("num_max_dispatch_tokens * num_topk exceeds int32")


MAX_ROW_ALIGN = 1024


def check_padding(num_topk: int, num_max_dispatch_tokens: int, num_experts: int, row_align: int,
                  expert_capacity: int) -> int:
    """Rules of the aligned / capacity-padded receive arrangements (limits
    chosen here: the pages fix none).  Returns the receive rows."""
    if not (1 <= row_align <= MAX_ROW_ALIGN):
        raise ValueError("row_align must be in [1, 1024]")
    if expert_capacity < 0:
        raise ValueError("negative expert_capacity")
    if expert_capacity > 0 and row_align > 1:
        raise ValueError("expert_capacity and row_align > 1 are exclusive")
    if expert_capacity > 0:
        rows = num_experts * expert_capacity
    else:
        rows = num_max_dispatch_tokens * num_topk + num_experts * (row_align - 1)
    if rows > 2 ** 31 - 1:
        raise ValueError("receive rows exceed int32")
    return rows


def check_hidden(hidden: int, mode: str) -> None:
    if mode not in QUANT_MODES:
        raise ValueError(f"unknown quant mode {mode!r}")
    if hidden <= 0 or hidden % 32:
        raise ValueError("hidden must be a positive multiple of 32")
    if mode.startswith("fp8_b128") and hidden % 128:
        raise ValueError("the per-128 e4m3 modes need hidden % 128 == 0")


def check_flags(use_fp8: bool, use_ue8m0: bool, use_mxfp4: bool, round_scale: bool,
                return_recv_hook: bool) -> str:
    """Map the low_latency_dispatch flags to a mode ("Low-Latency Mode API",
    Parameters: use_ue8m0 and use_mxfp4 both require use_fp8; round_scale
    goes with use_ue8m0, whose e8m0 scales are powers of two already, so it
    changes nothing there and is refused without it)."""
    if return_recv_hook:
        raise NotImplementedError("return_recv_hook is not supported")
    if round_scale and not use_ue8m0:
        raise ValueError("round_scale is used together with use_ue8m0")
    if (use_ue8m0 or use_mxfp4) and not use_fp8:
        raise ValueError("use_ue8m0 / use_mxfp4 require use_fp8")
    if use_ue8m0 and use_mxfp4:
        raise ValueError("use_ue8m0 and use_mxfp4 are exclusive")
    if not use_fp8:
        return "none"
    if use_mxfp4:
        return "mxfp4"
    if use_ue8m0:
        return "mxfp8"
    return "int8_token"
