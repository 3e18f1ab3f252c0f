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
        return int(self.offsets[-1])


def layout(topk_idx: np.ndarray, num_experts: int, num_max_dispatch_tokens: int,
           cum_stats: np.ndarray | None = None) -> Layout:
    idx = np.asarray(topk_idx).astype(np.int64)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    T, k = idx.shape
    E = int(num_experts)
    max_rows = int(num_max_dispatch_tokens) * k
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    status = 1 if np.any((flat != -1) & ~valid) else 0

    count = np.zeros(E, dtype=np.int64)
    for e in flat[valid]:
        count[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + count[e]

    slot = np.full(T * k, -1, dtype=np.int32)
    row_src = np.full(max_rows, -1, dtype=np.int32)
    fill = np.zeros(E, dtype=np.int64)
    for f in range(T * k):
        if not valid[f]:
            continue
        e = flat[f]
        r = offsets[e] + fill[e]
        fill[e] += 1
        slot[f] = r
        row_src[r] = f

    if cum_stats is not None:
        cum_stats += count.astype(cum_stats.dtype)
    return Layout(T, k, E, max_rows, count, offsets, slot.reshape(T, k), row_src, status)
