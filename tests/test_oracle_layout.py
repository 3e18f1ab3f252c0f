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
