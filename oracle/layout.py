"""Routing layout of the oracle (test infrastructure only).

What it computes ("Low-Latency Mode API", Parameters ``topk_idx`` and
Return Values ``recv_count``; the expert histogram, exclusive scan and
stable token-order slot assignment of the hot path):

* ``count[e]``  -- how many (token, j) pairs chose expert ``e``; ``-1`` means
  no expert.  Duplicates within one token count once each (the pages are silent;
  each pair gets its own row).
* ``offsets``   -- exclusive prefix sum of ``count``; ``offsets[E]`` is the
  number of routed rows R.  Expert ``e`` owns rows
  ``[offsets[e], offsets[e] + count[e])`` of the compact receive buffer
  (the pages show both a flat and a per-expert padded form; compact
  expert-major rows are the reading taken).
* ``slot[t, j]`` -- the receive row of pair (t, j), or -1.  Rows of one
  expert are in ascending (t, j) order (stable token order, ties within a
  token by j).
* ``row_src[r]`` -- ``t * k + j`` of the pair stored in row r, -1 for
  ``r >= R``.
* ``status``    -- bit 0 set when some id lies outside [-1, E); such pairs
  are dropped as if they were -1 (the pages are silent on such ids).
* ``cum_stats`` -- ``cumulative_local_expert_recv_stats`` plus ``count``
  ("Low-Latency Mode API", Parameters).

The loop below is the definition itself: walk the pairs in (t, j) order and
hand each routed pair the next free row of its expert.

Two receive-row arrangements besides the compact one:

* ``row_align = A > 1`` -- every expert's block of rows starts at a multiple
  of A: ``offsets`` is the exclusive prefix sum of ``align_up(count[e], A)``
  (the per-expert alignment a grouped GEMM wants; "EP dispatch with unfused
  MXFP8 quantization", Tests: the grouped path pins a per-expert alignment).
* ``expert_capacity = C > 0`` -- expert e owns rows [e*C, (e+1)*C): the padded
  per-expert form of the combine input in "Low-Latency Mode API"
  (``low_latency_combine`` Parameters, ``x``).  Pairs past the C-th of an
  expert are dropped (slot -1) and set status bit 1; ``count`` reports the
  rows actually received (at most C) while ``cum_stats`` adds the full demand.

Rows not holding a pair (alignment or capacity padding, and rows past the
last used one) have ``row_src`` -1.

Parity: pinned by brute force against ``np.argsort(kind="stable")`` and
``np.bincount`` (library routines), by the invariants sum(count) == number
of valid ids and "slot is a bijection onto [0, R)", and by the worked
example of the "[feat] A5 deep fused moe" page (Testing: every one of 8
experts receives 24 tokens, 192 per rank), stored in
``tests/golden/a5_fused_counts.txt``.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Layout:
    num_tokens: int
    num_topk: int
    num_experts: int
    max_rows: int               # num_max_dispatch_tokens * num_topk
    count: np.ndarray           # int64 [E]
    offsets: np.ndarray         # int64 [E+1]
    slot: np.ndarray            # int32 [T, k]
    row_src: np.ndarray         # int32 [max_rows]
    status: int

    @property
    def num_rows(self) -> int:
        """Rows up to the end of the last expert's block (compact: R)."""
        return int(self.offsets[-1])

    def valid_rows(self) -> np.ndarray:
        """Indices of the rows that hold a pair."""
        return np.nonzero(self.row_src >= 0)[0]


def layout(topk_idx: np.ndarray, num_experts: int, num_max_dispatch_tokens: int,
           cum_stats: np.ndarray | None = None, row_align: int = 1, expert_capacity: int = 0) -> Layout:
    idx = np.asarray(topk_idx).astype(np.int64)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    if row_align < 1 or expert_capacity < 0:
        raise ValueError("row_align >= 1 and expert_capacity >= 0")
    if expert_capacity > 0 and row_align > 1:
        raise ValueError("expert_capacity and row_align > 1 are exclusive")
    T, k = idx.shape
    E = int(num_experts)
    if expert_capacity > 0:
        max_rows = E * int(expert_capacity)
    else:
        max_rows = int(num_max_dispatch_tokens) * k + E * (row_align - 1)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    status = 1 if np.any((flat != -1) & ~valid) else 0

    demand = np.zeros(E, dtype=np.int64)
    for e in flat[valid]:
        demand[e] += 1
    if expert_capacity > 0:
        count = np.minimum(demand, expert_capacity)
        block = np.full(E, expert_capacity, dtype=np.int64)
        if np.any(demand > expert_capacity):
            status |= 2
    else:
        count = demand.copy()
        block = (count + row_align - 1) // row_align * row_align
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + block[e]

    slot = np.full(T * k, -1, dtype=np.int32)
    row_src = np.full(max_rows, -1, dtype=np.int32)
    fill = np.zeros(E, dtype=np.int64)
    for f in range(T * k):
        if not valid[f]:
            continue
        e = flat[f]
        rank = fill[e]
        fill[e] += 1
        if expert_capacity > 0 and rank >= expert_capacity:
            continue
        r = offsets[e] + rank
        slot[f] = r
        row_src[r] = f

    if cum_stats is not None:
        cum_stats += demand.astype(cum_stats.dtype)
    return Layout(T, k, E, max_rows, count, offsets, slot.reshape(T, k), row_src, status)
