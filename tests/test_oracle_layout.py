"""Pins of the oracle's routing layout.

* brute force: row_src equals the stable argsort of the valid expert ids
  (``np.argsort(kind="stable")``), counts equal ``np.bincount``;
* invariants: sum(count) is the number of valid ids; slot is a bijection onto
  [0, R); row_src[slot[f]] == f;
* the worked example of the "[feat] A5 deep fused moe" page (Testing table):
  24 tokens over 8 experts with top-8 give 24 per expert, 192 in total.
"""

import os

import numpy as np
import pytest

from oracle import layout as L

GOLD = os.path.join(os.path.dirname(__file__), "golden", "a5_fused_counts.txt")


def _read_gold():
    lines = [ln.split() for ln in open(GOLD) if ln.strip() and not ln.startswith("#")]
    (T, k, E), counts, (total,) = [list(map(int, ln)) for ln in lines]
    return T, k, E, counts, total


def _brute(idx, E):
    flat = idx.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    keys = np.where(valid, flat, E)                     # invalid pairs sort last
    order = np.argsort(keys, kind="stable")
    R = int(valid.sum())
    return np.bincount(flat[valid], minlength=E), order[:R]


@pytest.mark.parametrize("seed", range(12))
def test_layout_matches_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(0, 60))
    k = int(rng.integers(1, 17))
    E = int(rng.integers(1, 40))
    idx = rng.integers(-1, E, size=(T, k))
    if seed % 3 == 0 and T:                             # some ids out of range
        idx[rng.integers(0, T), rng.integers(0, k)] = E + 3
        idx[rng.integers(0, T), rng.integers(0, k)] = -7
    lay = L.layout(idx, E, T + 5)
    cnt, rows = _brute(idx, E)
    assert np.array_equal(lay.count, cnt)
    R = lay.num_rows
    assert R == rows.size
    assert np.array_equal(lay.row_src[:R], rows)
    assert np.all(lay.row_src[R:] == -1)
    bad = np.any((idx != -1) & ((idx < 0) | (idx >= E)))
    assert lay.status == int(bad)


@pytest.mark.parametrize("seed", range(6))
def test_layout_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    T, k, E = 300, 8, 32
    idx = rng.integers(-1, E, size=(T, k))
    lay = L.layout(idx, E, T)
    valid = idx.reshape(-1) >= 0
    assert lay.count.sum() == valid.sum() == lay.num_rows
    s = lay.slot.reshape(-1)
    assert np.all(s[~valid] == -1)
    assert np.array_equal(np.sort(s[valid]), np.arange(lay.num_rows))
    assert np.all(lay.row_src[s[valid]] == np.nonzero(valid)[0])
    # expert e owns rows [offsets[e], offsets[e+1])
    for f in np.nonzero(valid)[0]:
        e = idx.reshape(-1)[f]
        assert lay.offsets[e] <= s[f] < lay.offsets[e + 1]


def test_layout_duplicates_get_their_own_rows():
    idx = np.array([[3, 3, 1], [1, -1, 3]])
    lay = L.layout(idx, 4, 2)
    assert list(lay.count) == [0, 2, 0, 3]
    assert lay.slot.tolist() == [[2, 3, 0], [1, -1, 4]]


def test_layout_worked_example_from_pages():
    T, k, E, counts, total = _read_gold()
    rng = np.random.default_rng(7)
    idx = np.stack([rng.permutation(E) for _ in range(T)])[:, :k]
    lay = L.layout(idx, E, T)
    assert lay.count.tolist() == counts
    assert lay.num_rows == total == sum(counts)


def test_layout_empty_and_all_negative():
    lay = L.layout(np.zeros((0, 4), np.int64), 8, 16)
    assert lay.num_rows == 0 and lay.row_src.size == 64 and np.all(lay.row_src == -1)
    lay = L.layout(-np.ones((5, 3), np.int64), 8, 5)
    assert lay.num_rows == 0 and np.all(lay.slot == -1)


def test_layout_cumulative_stats():
    idx = np.array([[0, 1], [1, 1]])
    cum = np.array([5, 0, 2], np.int32)
    L.layout(idx, 3, 2, cum_stats=cum)
    assert cum.tolist() == [6, 3, 2]


# ---------------------------------------------------------------------------
# aligned and capacity-padded per-expert arrangements
# ---------------------------------------------------------------------------


def _brute_padded(idx, E, tmax, align=1, cap=0):
    """Expected (count, offsets, row_src, slot, status) from the stable
    argsort: expert e's pairs in (t, j) order, placed at the start of its
    block (blocks of align_up(count, align) rows, or of cap rows)."""
    T, k = idx.shape
    demand, order = _brute(idx, E)
    starts_compact = np.concatenate([[0], np.cumsum(demand)])
    if cap:
        blocks = np.full(E, cap)
        max_rows = E * cap
    else:
        blocks = -(-demand // align) * align
        max_rows = tmax * k + E * (align - 1)
    offsets = np.concatenate([[0], np.cumsum(blocks)])
    row_src = np.full(max_rows, -1)
    slot = np.full(T * k, -1)
    for e in range(E):
        mine = order[starts_compact[e]:starts_compact[e + 1]]
        if cap:
            mine = mine[:cap]
        rows = offsets[e] + np.arange(mine.size)
        row_src[rows] = mine
        slot[mine] = rows
    flat = idx.reshape(-1)
    status = int(np.any((flat != -1) & ((flat < 0) | (flat >= E))))
    if cap and np.any(demand > cap):
        status |= 2
    count = np.minimum(demand, cap) if cap else demand
    return count, offsets, row_src, slot.reshape(T, k), status, demand


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("align", [1, 2, 8, 128])
def test_aligned_layout_matches_brute(seed, align):
    rng = np.random.default_rng(500 + seed)
    T = int(rng.integers(0, 50))
    k = int(rng.integers(1, 17))
    E = int(rng.integers(1, 30))
    idx = rng.integers(-1, E, size=(T, k))
    if seed % 4 == 1 and T:
        idx[0, 0] = E + 1
    stats = np.zeros(E, np.int64)
    lay = L.layout(idx, E, T + 3, cum_stats=stats, row_align=align)
    count, offsets, row_src, slot, status, demand = _brute_padded(idx, E, T + 3, align=align)
    assert lay.max_rows == row_src.size
    assert np.array_equal(lay.count, count)
    assert np.array_equal(lay.offsets, offsets)
    assert np.all(lay.offsets % align == 0)
    assert np.array_equal(lay.row_src, row_src)
    assert np.array_equal(lay.slot, slot)
    assert lay.status == status
    assert np.array_equal(stats, demand)
    assert lay.num_rows <= lay.max_rows


@pytest.mark.parametrize("seed", range(10))
def test_capacity_layout_matches_brute(seed):
    rng = np.random.default_rng(700 + seed)
    T = int(rng.integers(1, 50))
    k = int(rng.integers(1, 9))
    E = int(rng.integers(1, 20))
    idx = rng.integers(-1, E, size=(T, k))
    demand = np.bincount(idx[idx >= 0], minlength=E)
    cap = int(rng.integers(1, demand.max() + 3)) if demand.max() > 0 else 1
    stats = np.zeros(E, np.int64)
    lay = L.layout(idx, E, T, cum_stats=stats, expert_capacity=cap)
    count, offsets, row_src, slot, status, dem = _brute_padded(idx, E, T, cap=cap)
    assert lay.max_rows == E * cap
    assert np.array_equal(lay.count, count)
    assert np.array_equal(lay.offsets, offsets)
    assert np.array_equal(lay.row_src, row_src)
    assert np.array_equal(lay.slot, slot)
    assert lay.status == status
    assert np.array_equal(stats, dem)          # statistics count the whole demand


def test_align_one_and_large_capacity_reduce_to_compact():
    rng = np.random.default_rng(9)
    idx = rng.integers(-1, 12, size=(40, 6))
    base = L.layout(idx, 12, 40)
    same = L.layout(idx, 12, 40, row_align=1)
    assert np.array_equal(base.slot, same.slot) and np.array_equal(base.row_src, same.row_src)
    # capacity >= every demand: the slot of a pair is e*C + (its compact row - offsets[e])
    C = int(base.count.max())
    padded = L.layout(idx, 12, 40, expert_capacity=C)
    assert padded.status == 0
    flat, s0, s1 = idx.reshape(-1), base.slot.reshape(-1), padded.slot.reshape(-1)
    ok = flat >= 0
    assert np.array_equal(s1[ok], flat[ok] * C + (s0[ok] - base.offsets[flat[ok]]))
    assert np.all(s1[~ok] == -1)


def test_padded_layouts_worked_example():
    # two tokens, top-3, four experts: expert 1 gets pairs (0,2), (1,0);
    # expert 3 gets (0,0), (0,1), (1,2), in that order
    idx = np.array([[3, 3, 1], [1, -1, 3]])
    a = L.layout(idx, 4, 2, row_align=4)
    assert a.offsets.tolist() == [0, 0, 4, 4, 8]
    assert a.slot.tolist() == [[4, 5, 0], [1, -1, 6]]
    assert a.row_src.tolist()[:8] == [2, 3, -1, -1, 0, 1, 5, -1]
    assert a.max_rows == 2 * 3 + 4 * 3
    c = L.layout(idx, 4, 2, expert_capacity=2)
    assert c.offsets.tolist() == [0, 2, 4, 6, 8]
    assert c.slot.tolist() == [[6, 7, 2], [3, -1, -1]]
    assert c.row_src.tolist() == [-1, -1, 2, 3, -1, -1, 0, 1]
    assert c.count.tolist() == [0, 2, 0, 2]
    assert c.status == 2


def test_padded_layout_rejects_bad_arguments():
    idx = np.zeros((2, 2), np.int64)
    with pytest.raises(ValueError):
        L.layout(idx, 4, 2, row_align=0)
    with pytest.raises(ValueError):
        L.layout(idx, 4, 2, expert_capacity=-1)
