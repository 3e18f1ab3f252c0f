"""Test helper: the oracle's dispatch of a whole full-size workload, with
its one costly step -- ``oracle.quant.quantize_row`` of each token row,
about 10 ms per 7168-wide row -- spread over worker processes.

``dispatch_parallel`` returns what ``oracle.dispatch.dispatch`` returns: every
token row is quantised once by the oracle's own row quantiser (in a worker)
and written to each receive row its routed pairs hold, as ``dispatch`` does;
``tests/test_oracle_path.py`` checks the two agree.  Workers are started
with "spawn" and import only numpy and ``oracle``, so nothing of the GPU
process is copied into them.  Results are cached per workload for the test
session (the full-size tests of several files share one input set)."""

from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import dispatch as D, quant as Q
from oracle.layout import Layout

_CACHE: dict = {}


def _quantize_rows(args):
    mode, rows = args
    out_d, out_s = [], []
    for r in rows:
        d, s = Q.quantize_row(mode, r)
        out_d.append(d)
        out_s.append(s)
    return np.stack(out_d), np.stack(out_s)


def quantize_all(mode: str, x_bits: np.ndarray, workers: int | None = None, chunk: int = 128):
    """(codes [T, Dq], scales [T, Sq]) of every token row, by the oracle's
    quantize_row; cached for the session under a digest of the rows."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    key = (mode, x_bits.shape, hashlib.blake2b(x_bits.tobytes(), digest_size=16).hexdigest())
    if key in _CACHE:
        return _CACHE[key]
    T = x_bits.shape[0]
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    tasks = [(mode, x_bits[i:i + chunk]) for i in range(0, T, chunk)]
    if workers == 1 or len(tasks) <= 1:
        parts = [_quantize_rows(t) for t in tasks]
    else:
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            parts = list(ex.map(_quantize_rows, tasks))
    dq, sq = Q.row_bytes(mode, x_bits.shape[1])
    codes = np.concatenate([p[0] for p in parts]) if parts else np.zeros((0, dq), np.uint8)
    scales = np.concatenate([p[1] for p in parts]) if parts else np.zeros((0, sq), np.uint8)
    _CACHE[key] = (codes, scales)
    return codes, scales


def dispatch_parallel(x_bits: np.ndarray, lay: Layout, mode: str, workers: int | None = None) -> D.RecvBuffer:
    """The oracle's dispatch (without receive weights), rows quantised in
    worker processes: every routed pair (t, j) writes token t's codes and
    scales to row slot[t, j]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    dq, sq = Q.row_bytes(mode, H)
    codes, scales = quantize_all(mode, x_bits, workers)
    data = np.zeros((lay.max_rows, dq), np.uint8)
    sc = np.zeros((lay.max_rows, sq), np.uint8)
    for t in range(T):
        for j in range(lay.num_topk):
            r = int(lay.slot[t, j])
            if r >= 0:
                data[r] = codes[t]
                sc[r] = scales[t]
    return D.RecvBuffer(mode, H, lay.num_rows, data, sc, None)


def _backward_rows(args):
    from oracle import backward as B
    mode, rows, weights = args
    out_d, out_s = [], []
    for r, w in zip(rows, weights):
        d, s = Q.quantize_row(mode, r if w is None else B.scaled_grad_row(r, w))
        out_d.append(d)
        out_s.append(s)
    return out_d, out_s


def backward_parallel(grad_bits: np.ndarray, lay: Layout, mode: str, topk_weights: np.ndarray | None,
                      tokens, workers: int | None = None, chunk: int = 256) -> dict:
    """The oracle's combine backward for the listed tokens: {row: (codes,
    scales)} for every routed pair, each row quantised in a worker by the
    oracle's own steps (``backward.scaled_grad_row`` with the pair's weight,
    then ``quant.quantize_row``), as ``backward.combine_backward`` does."""
    grad_bits = np.asarray(grad_bits, dtype=np.uint16)
    pairs = [(int(t), j, int(lay.slot[t, j])) for t in tokens for j in range(lay.num_topk) if lay.slot[t, j] >= 0]
    tasks = []
    for i in range(0, len(pairs), chunk):
        part = pairs[i:i + chunk]
        rows = np.stack([grad_bits[t] for t, _, _ in part]) if part else np.zeros((0, grad_bits.shape[1]), np.uint16)
        ws = [None if topk_weights is None else float(topk_weights[t, j]) for t, j, _ in part]
        tasks.append((mode, rows, ws))
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    if workers == 1 or len(tasks) <= 1:
        parts = [_backward_rows(t) for t in tasks]
    else:
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            parts = list(ex.map(_backward_rows, tasks))
    out = {}
    it = iter(pairs)
    for ds, ss in parts:
        for d, s in zip(ds, ss):
            _, _, r = next(it)
            out[r] = (d, s)
    return out
