"""Benchmark of MoE dispatch + combine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--row-align A | --expert-capacity C]

One step is one pass of the whole path over one batch: ep_layout (routing
layout), ep_dispatch (quantise + scatter) and ep_combine (gather + dequantise
+ weighted reduce), all launched on one stream with inputs resident in HBM.
Buffer sets rotate between steps so that no step finds its inputs in the
256 MB last-level cache.  The default workload is "large": 16384 tokens,
hidden 7168, top-8 of 256 experts with 5% of the pairs unrouted, MXFP4
dispatch and a bf16 combine.  --row-align / --expert-capacity time the same
workload on aligned or capacity-padded expert blocks (ep_layout_ex).

Prints one JSON line: tokens/s over the timed steps, the algorithmic bytes
and GB/s of the whole step, the roofline entry of the dominant kernel
(combine) with its duration measured by HIP events on the launch stream, and
the CPU oracle's throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), H=7168 k=8"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_large_traffic.json")
KERNEL_SOURCES = ["combine_topk_idx_amd/csrc/combine.hip", "combine_topk_idx_amd/csrc/formats.hpp",
                  "combine_topk_idx_amd/csrc/common.hpp"]
MOE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gmm1_moe_share_traffic.json")
MOE_KERNEL_SOURCES = ["combine_topk_idx_amd/csrc/moe.hip", "combine_topk_idx_amd/csrc/moe.hpp",
                      "combine_topk_idx_amd/csrc/formats.hpp", "combine_topk_idx_amd/csrc/common.hpp"]


def algorithmic_bytes(w, R: int) -> dict:
    """Bytes the method has to move, per phase.

    layout:   read ids, write counts/offsets, slot map and row sources
    dispatch: read x once and the slot map, write every routed packed row
    combine:  read every routed row, the ids and the weights, write out
    """
    b_idx = 4 if w.idx_dtype == "int32" else 8
    H, T, k, E = w.H, w.T, w.k, w.E
    dq, sq = _row_bytes(w.mode, H)
    cin = w.mode if w.combine_input == "identity" else "none"   # scaled_dispatch: bf16 rows
    dc, sc = _row_bytes(cin, H)
    lay = T * k * b_idx + E * 8 + (E + 1) * 4 + T * k * 4 + R * 4
    disp = 2 * T * H + T * k * 4 + R * (dq + sq)
    comb = R * (dc + sc) + T * k * (b_idx + 4) + 2 * T * H
    return {"layout": lay, "dispatch": disp, "combine": comb, "total": lay + disp + comb}


def _row_bytes(mode: str, H: int):
    return {"none": (2 * H, 0), "int8_token": (H, 4), "fp8_b128": (H, 4 * (H // 128)),
            "fp8_b128_pow2": (H, 4 * (H // 128)), "fp8_b128_ue8m0": (H, H // 128),
            "mxfp8": (H, H // 32), "mxfp4": (H // 2, H // 32)}[mode]


def _source_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernel sources' code: comments and whitespace are left
    out, so that a comment edit does not retire measured counters."""
    import re
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, path: str = TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the measured kernel from a committed rocprofv3
    counter summary, or None if it is missing, for another workload, or was
    taken on a different kernel source."""
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != _source_hash(sources) or d.get("workload") != workload:
        return None
    return d.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU oracle leg (runs in a child process pinned to one core)
# ---------------------------------------------------------------------------


CPU_RUNS = 3             # timed oracle runs of the sample; the median is reported
CPU_ONE_RUN_S = 60.0     # ... or one run, when a run takes longer than this


def _timed_runs(run) -> list:
    """Times `run()` CPU_RUNS times, or once if that run exceeds CPU_ONE_RUN_S."""
    times = []
    for _ in range(CPU_RUNS):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        if times[0] > CPU_ONE_RUN_S:
            break
    return times


def cpu_baseline_child(name: str, tokens: int) -> None:
    """The oracle's layout + dispatch + combine on the first `tokens` tokens
    as one batch, on one core, timed CPU_RUNS times (inputs drawn once,
    outside the timed region)."""
    os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    import numpy as np
    from combine_topk_idx_amd import workloads as W
    from oracle import combine as C, dispatch as D, layout as L

    w = W.WORKLOADS[name]
    inp = W.make_inputs(w)
    x = inp["x"][:tokens]
    idx = inp["topk_idx"][:tokens]
    wts = inp["topk_weights"][:tokens]
    y = None
    if w.combine_input == "normal":
        y = W.make_expert_out(w, rows=tokens * w.k)

    def run():
        lay = L.layout(idx, w.E, tokens)
        rb = D.dispatch(x, lay, w.mode)
        if w.combine_input == "identity":
            cin = rb
        elif w.combine_input == "scaled_dispatch":                # bf16 rows: the dispatched rows x 1.5
            from oracle import codecs
            ys = codecs.bf16_bits_to_f32(rb.data.view(np.uint16)).astype(np.float32) * np.float32(1.5)
            cin = D.RecvBuffer("none", w.H, lay.num_rows, W.bf16_from_f32(ys).view(np.uint8),
                               np.zeros((lay.max_rows, 0), np.uint8), None)
        else:
            cin = D.RecvBuffer("none", w.H, lay.num_rows, y.view(np.uint8).reshape(tokens * w.k, -1),
                               np.zeros((tokens * w.k, 0), np.uint8), None)
        C.combine(cin, lay, wts)

    times = _timed_runs(run)
    print(json.dumps({"tokens": tokens, "times": times, "cores": len(os.sched_getaffinity(0))}))


def cpu_baseline_moe_child(name: str, tokens: int) -> None:
    """The oracle's expert-MLP path (layout, MXFP8 dispatch, GMM1 + SwiGLU +
    requant, GMM2, combine) on the first `tokens` tokens, on one core, timed
    CPU_RUNS times."""
    os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    import numpy as np
    from combine_topk_idx_amd import workloads as W
    from oracle import combine as C, dispatch as D, layout as L, moe as M

    w = W.MOE_WORKLOADS[name]
    inp = W.make_moe_inputs(w)
    x, idx, wts = inp["x"][:tokens], inp["topk_idx"][:tokens], inp["topk_weights"][:tokens]
    rows_seen = []

    def run():
        lay = L.layout(idx, w.E_local, tokens)
        rb = D.dispatch(x, lay, "mxfp8")
        y = np.zeros((lay.max_rows, w.H), np.uint16)
        for e in range(w.E_local):
            rows = np.arange(lay.offsets[e], lay.offsets[e] + lay.count[e])
            if rows.size == 0:
                continue
            q, qs, _ = M.gmm1_swiglu_rows(rb.data[rows], rb.scales[rows], inp["w1_codes"][e], inp["w1_scales"][e])
            y[rows], _ = M.gmm2_rows(q, qs, inp["w2_codes"][e], inp["w2_scales"][e])
        cin = D.RecvBuffer("none", w.H, lay.num_rows, y.view(np.uint8), np.zeros((lay.max_rows, 0), np.uint8),
                           None)
        C.combine(cin, lay, wts)
        rows_seen.append(int(lay.num_rows))

    times = _timed_runs(run)
    print(json.dumps({"tokens": tokens, "rows": rows_seen[0], "times": times,
                      "cores": len(os.sched_getaffinity(0))}))


def cpu_baseline(name: str, tokens: int, moe: bool = False) -> dict:
    flag = "--cpu-baseline-moe-child" if moe else "--cpu-baseline-child"
    r = subprocess.run([sys.executable, os.path.abspath(__file__), flag, name,
                        "--cpu-tokens", str(tokens)], capture_output=True, text=True, env=dict(
                            os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
                            HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES=""))
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline failed:\n{r.stderr}")
    d = json.loads(r.stdout.strip().splitlines()[-1])
    times = sorted(d["times"])
    med = times[len(times) // 2]
    what = ("layout + MXFP8 dispatch + GMM1/SwiGLU/requant + GMM2 + combine, "
            f"{d.get('rows', 0)} expert rows; the weights are dequantised in full" if moe else
            "layout + dispatch + combine")
    runs = (f"median of {len(times)} runs ({', '.join(f'{t:.2f}' for t in d['times'])} s)" if len(times) > 1
            else f"one run of {times[0]:.1f} s (over {CPU_ONE_RUN_S:.0f} s)")
    return {"value": d["tokens"] / med, "unit": "tokens/s", "cores": d["cores"], "kind": "oracle",
            "sample": f"first {d['tokens']} tokens of the workload as one batch ({what}), {runs}, "
                      f"on one host core",
            "seconds": round(med, 3), "host": _host_cpu()}


def _host_cpu() -> str:
    """'1 core of N <model>' for the host the oracle ran on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"1 core of {len(os.sched_getaffinity(0))} ({model})"


# ---------------------------------------------------------------------------
# GPU leg
# ---------------------------------------------------------------------------


def timed_steps(runners, steps: int, stream):
    """Throughput pass: `steps` steps (runners[i % len] is the list of phase
    calls of step i) between one event before the first and one after the
    last, nothing in between, synchronised on both sides.  Then a phase
    pass: the same steps again with an event between consecutive phases
    (an event on the stream takes a few microseconds of its own, so the
    throughput pass has none).  Returns (ms per step, [ms per phase],
    wall seconds of the throughput pass, {p10, p50, p90} of the per-step
    times of the phase pass, events included)."""
    import torch
    nph = len(runners[0])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        for f in runners[i % len(runners)]:
            f()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        for j, f in enumerate(runners[i % len(runners)]):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    ph = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j in range(nph)]
    per = sorted(e[0].elapsed_time(e[nph]) for e in ev)
    pick = lambda q: per[min(len(per) - 1, int(q * len(per)))]
    dist = {"p10": round(pick(0.1), 5), "p50": round(pick(0.5), 5), "p90": round(pick(0.9), 5)}
    return ms, ph, wall, dist


def graph_steps(runners, steps: int, stream) -> float:
    """The same `steps` steps captured once into one HIP graph (every phase
    call of every step a kernel node, on the rotating buffer sets), replayed
    once untimed and then once between two events on `stream`: the GPU's
    time per step without the host's per-call launch cost.  Returns ms per
    step."""
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            for f in runners[i % len(runners)]:
                f()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def probes_main(args) -> int:
    """Floors and ceilings of the path's access patterns, from the probe
    kernels of libep_probe.so (an empty grid, combine's gather with no
    dequantisation, 16-byte streams); one JSON line.  Decode-sized probes are
    timed as graph replays over rotating buffer sets (cache-cold, no host
    cost per launch), the large ones as stream launches between events."""
    import ctypes
    import numpy as np
    import torch
    from combine_topk_idx_amd import build as B

    lib = ctypes.CDLL(B.PROBE_LIB)
    vp = ctypes.c_void_p
    lib.ep_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, vp]
    lib.ep_probe_gather.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.ep_probe_stream.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int, vp]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cur = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

    def ok(rc):
        if rc != 0:
            raise RuntimeError("probe launch failed")

    def graph_ms(calls, reps):
        """ms per call: `reps` calls (rotating over `calls`) in one graph."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                calls[i % len(calls)]()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def stream_ms(call, reps):
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    T, k, H, rows = 128, 8, 7168, 1024                 # the decode workload: 896 span workgroups
    chunks = (H // 8 + 127) // 128
    for name, blocks in (("empty_1wg", 1), ("empty_decode_combine_grid", T * chunks),
                         ("empty_decode_layout_dispatch_grid", T * chunks + 1)):
        res[name] = {"us": round(1e3 * graph_ms([lambda b=blocks: ok(lib.ep_probe_empty(b, 128, cur()))], 200), 3),
                     "grid": blocks}
    rng = np.random.default_rng(7)
    nsets = 42                                       # > 1 GB of rows over the sets, as the decode bench
    sets = []
    for _ in range(nsets):
        sl = rng.permutation(rows)[: T * k].astype(np.int32)
        sl[rng.choice(T * k, size=round(0.1 * T * k), replace=False)] = -1
        sets.append({"rows": torch.empty((rows, H), dtype=torch.bfloat16, device=dev).normal_(),
                     "slot": torch.from_numpy(sl).to(dev),
                     "slot1": torch.from_numpy(sl.reshape(T, k)[:, :1].copy()).to(dev),
                     "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)})
    for kk in (1, 8):
        calls = [lambda s=s, kk=kk: ok(lib.ep_probe_gather(s["rows"].data_ptr(), s["slot" if kk == 8 else "slot1"]
                                                           .data_ptr(), T, kk, H, s["out"].data_ptr(), cur()))
                 for s in sets]
        ms = graph_ms(calls, 210)
        R = int((sets[0]["slot"] >= 0).sum()) if kk == 8 else T
        nbytes = R * 2 * H + T * kk * 4 + 2 * T * H
        res[f"gather_decode_k{kk}"] = {"us": round(1e3 * ms, 3), "bytes": nbytes,
                                       "gbps": round(nbytes / ms / 1e6, 1)}
    # dispatch's pattern at decode: each token's span read once and written
    # as one byte per element to each of its routed rows
    lib.ep_probe_scatter.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    for s in sets:
        s["x"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev).normal_()
        s["codes"] = s["rows"].view(-1).view(torch.uint8)[: rows * H].view(rows, H)
    for kk in (1, 8):
        calls = [lambda s=s, kk=kk: ok(lib.ep_probe_scatter(s["x"].data_ptr(), s["slot" if kk == 8 else "slot1"]
                                                            .data_ptr(), T, kk, H, s["codes"].data_ptr(), cur()))
                 for s in sets]
        ms = graph_ms(calls, 210)
        R = int((sets[0]["slot"] >= 0).sum()) if kk == 8 else T
        nbytes = 2 * T * H + T * kk * 4 + R * H
        res[f"scatter_decode_k{kk}"] = {"us": round(1e3 * ms, 3), "bytes": nbytes,
                                        "gbps": round(nbytes / ms / 1e6, 1)}
    del sets
    torch.cuda.empty_cache()
    # the large workload's combine pattern: 16384 tokens, 8 random rows each
    T, rows = 16384, 131072
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev).normal_()
    sl = rng.permutation(rows).astype(np.int32)
    sl[rng.choice(rows, size=round(0.05 * rows), replace=False)] = -1
    slot = torch.from_numpy(sl).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ms = stream_ms(lambda: ok(lib.ep_probe_gather(y.data_ptr(), slot.data_ptr(), T, 8, H, out.data_ptr(), cur())), 20)
    R = int((slot >= 0).sum())
    nbytes = R * 2 * H + T * 8 * 4 + 2 * T * H
    res["gather_large_k8"] = {"us": round(1e3 * ms, 2), "bytes": nbytes, "gbps": round(nbytes / ms / 1e6, 1)}
    del y, out
    torch.cuda.empty_cache()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for mode, name, moved in ((0, "read_1GiB", n), (1, "write_1GiB", n), (2, "copy_1GiB", 2 * n)):
        best = None
        for blocks in (1024, 2048, 4096, 8192, 16384, 65536):   # the best grid of each stream
            ms = stream_ms(lambda m=mode, b=blocks: ok(lib.ep_probe_stream(m, src.data_ptr(), dst.data_ptr(), n, b,
                                                                           cur())), 10)
            if best is None or ms < best[0]:
                best = (ms, blocks)
        ms, blocks = best
        res[name] = {"us": round(1e3 * ms, 1), "bytes": moved, "gbps": round(moved / ms / 1e6, 1), "grid": blocks}
    del dst
    # the expert GEMMs' weight stream: every wave its own contiguous range in
    # 2 KB steps, 4 or 8 steps in flight, one workgroup per CU (or two)
    lib.ep_probe_wave_stream.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                         vp]
    wout = torch.empty((4096, 16), dtype=torch.uint8, device=dev)
    span = 512 << 20                                   # beyond the 256 MB last-level cache
    for blocks, waves, depth, one in ((256, 6, 4, 1), (256, 6, 8, 1), (240, 6, 4, 1), (192, 6, 4, 1), (48, 6, 4, 1),
                                      (256, 8, 4, 1), (256, 4, 4, 1), (512, 4, 4, 0), (512, 6, 4, 0)):
        steps = span // (blocks * waves * 2048) // depth * depth
        moved = blocks * waves * steps * 2048
        ms = stream_ms(lambda b=blocks, wv=waves, st=steps, d=depth, o=one: ok(lib.ep_probe_wave_stream(
            src.data_ptr(), b, wv, st, d, o, wout.data_ptr(), cur())), 10)
        cus = blocks if one else blocks // 2
        res[f"wave_stream_{blocks}x{waves}_d{depth}" + ("" if one else "_2perCU")] = {
            "us": round(1e3 * ms, 1), "bytes": moved, "gbps": round(moved / ms / 1e6, 1),
            "gbps_per_cu": round(moved / ms / 1e6 / cus, 1)}
    # the GEMMs' whole fetch per CU: the weight stream plus 12 KB of shared
    # activations per step (two 16-byte pieces per thread), from L2
    lib.ep_probe_mixed_stream.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    act = torch.empty(1 << 20, dtype=torch.uint8, device=dev).fill_(3)
    for blocks in (240, 256):
        waves, depth = 6, 4
        steps = span // (blocks * waves * 2048) // depth * depth
        wbytes = blocks * waves * steps * 2048
        abytes = blocks * waves * 64 * steps * 2 * 16
        ms = stream_ms(lambda b=blocks, st=steps: ok(lib.ep_probe_mixed_stream(
            src.data_ptr(), act.data_ptr(), act.numel(), b, waves, st, wout.data_ptr(), cur())), 10)
        res[f"mixed_stream_{blocks}x{waves}"] = {
            "us": round(1e3 * ms, 1), "weight_bytes": wbytes, "activation_bytes": abytes,
            "weight_gbps": round(wbytes / ms / 1e6, 1), "gbps_per_cu": round((wbytes + abytes) / ms / 1e6 / blocks, 1)}
    # the matrix cores: back-to-back independent instructions on every wave,
    # one workgroup per CU; a SIMD carries ceil(waves / 4) of them
    lib.ep_probe_mfma_rate.argtypes = [ctypes.c_int] * 6 + [vp, vp]
    mout = torch.empty(256 * 8 * 64, dtype=torch.float32, device=dev)
    iters = 1000
    for kind, name, flop, chains in ((0, "mx_e4m3_32x32x64", 2 * 32 * 32 * 64, 8),
                                     (0, "mx_e4m3_32x32x64_4chains", 2 * 32 * 32 * 64, 4),
                                     (1, "bf16_32x32x16", 2 * 32 * 32 * 16, 8)):
        for waves in (4, 6, 8):
            ms = stream_ms(lambda k=kind, c=chains, wv=waves: ok(lib.ep_probe_mfma_rate(k, c, 256, wv, iters, 1,
                                                                                        mout.data_ptr(), cur())), 5)
            per_simd = -(-waves // 4) * iters * 8
            res[f"mfma_{name}_{waves}waves"] = {
                "us": round(1e3 * ms, 1), "tflops": round(256 * waves * iters * 8 * flop / ms / 1e9, 1),
                "ns_per_instr_per_simd": round(1e6 * ms / per_simd, 2)}
    print(json.dumps({"probes": res, "peak_gbps": HBM_PEAK_GBPS}), flush=True)
    return 0


def backward_main(args) -> int:
    """layout + ep_combine_backward on one workload's routing; one JSON line."""
    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    from combine_topk_idx_amd import ep, workloads as W

    w = W.WORKLOADS[args.workload]
    q = args.combine_backward
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w)
    grad = W.make_expert_out(w, rows=w.T)
    total, _ = ep.ep_buffer_bytes(w.max_rows, w.H, q)
    nsets = args.sets or max(2, -(-(1 << 30) // max(4 * w.T * w.H + total, 1)))
    sets = [dict(idx=torch.from_numpy(inp["topk_idx"]).to(dev), w=torch.from_numpy(inp["topk_weights"]).to(dev),
                 g=torch.from_numpy(grad.view(np.int16)).to(dev).view(torch.bfloat16),
                 ws=torch.empty(ep.ep_workspace_bytes(w.t_max, w.k, w.E), dtype=torch.uint8, device=dev),
                 rc=torch.empty(w.E, dtype=torch.int64, device=dev),
                 buf=torch.empty(total, dtype=torch.uint8, device=dev)) for _ in range(min(nsets, 64))]
    stream = torch.cuda.current_stream()

    def lay(s):
        s["h"] = ep.ep_layout(s["idx"], w.E, w.t_max, s["rc"], s["ws"])

    def bwd(s):
        ep.ep_combine_backward(s["h"], s["g"], w.H, q, s["buf"], s["w"])

    for i in range(max(args.warmup, len(sets))):
        lay(sets[i % len(sets)])
        bwd(sets[i % len(sets)])
    torch.cuda.synchronize()
    R = int(sets[0]["rc"].sum().item())
    runners = [[(lambda s=s: lay(s)), (lambda s=s: bwd(s))] for s in sets]
    ms, (lay_ms, bwd_ms), _, dist = timed_steps(runners, args.steps, stream)
    dq, sqb = _row_bytes(q, w.H)
    b_idx = 4 if w.idx_dtype == "int32" else 8
    b_lay = w.T * w.k * b_idx + w.E * 8 + (w.E + 1) * 4 + w.T * w.k * 4 + R * 4
    b_bwd = 2 * w.T * w.H + w.T * w.k * 8 + R * (dq + sqb)
    gbps = (b_lay + b_bwd) / (ms * 1e-3) / 1e9
    bwd_gbps = b_bwd / (bwd_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "combine-backward reverse dispatch tokens/s and achieved HBM GB/s (% of peak), H=7168 k=8",
        "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name} routing: T={w.T} H={w.H} E={w.E} k={w.k}, weighted gradient rows "
                               f"quantised to {q}", "T": w.T, "H": w.H, "E": w.E, "k": w.k, "rows": R},
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "phase_ms": {"layout": round(lay_ms, 5), "combine_backward": round(bwd_ms, 5)},
        "step_ms_phase_pass": dist,
        "roofline": {"bound": "hbm", "kernel": "combine_backward", "achieved": round(bwd_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "alg_bytes_per_launch": b_bwd, "avg_launch_ms": round(bwd_ms, 5)},
        "cpu_baseline": None}), flush=True)
    return 0


MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 / MXFP8 matrix-core peak


def moe_algorithmic(w, R: int) -> dict:
    """Bytes and flops of the expert-MLP path for R routed rows.

    dispatch: read the x rows of routed tokens (at most T), write R MXFP8 rows
    gmm1:     read W1 (codes + scales, packed once ahead of time) and the R
              dispatch rows, write R MXFP8 rows of width I
    gmm2:     read W2 (codes + scales) and those rows, write R bf16 rows
    combine:  read R bf16 rows, the (int64) ids and the weights, write T bf16 rows
    """
    H, I, E, T, k = w.H, w.I, w.E_local, w.T, w.k
    mx = lambda n: n + n // 32
    b = {
        "layout": T * k * 8 + E * 8 + (E + 1) * 4 + T * k * 4 + R * 4,
        "dispatch": 2 * T * H + T * k * 4 + R * mx(H),
        "gmm1": E * 2 * I * mx(H) + R * mx(H) + R * mx(I),
        "gmm2": E * H * mx(I) + R * mx(I) + R * 2 * H,
        "combine": R * 2 * H + T * k * (8 + 4) + 2 * T * H,
    }
    b["total"] = sum(b.values())
    f = {"gmm1": 2.0 * R * H * 2 * I, "gmm2": 2.0 * R * I * H}
    return {"bytes": b, "flops": f}


def moe_main(args) -> int:
    """layout + MXFP8 dispatch + GMM1/SwiGLU/requant + GMM2 + combine of one
    MoE workload; one JSON line."""
    import numpy as np
    import torch
    from combine_topk_idx_amd import ep, workloads as W

    w = W.MOE_WORKLOADS[args.moe]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}: T={w.T} H={w.H} I={w.I} E={w.E_local}/{w.E_total} k={w.k}",
          file=sys.stderr, flush=True)
    inp = W.make_moe_inputs(w)
    rows = w.max_rows
    xb, _ = ep.ep_buffer_bytes(rows, w.H, "mxfp8")
    ab, _ = ep.ep_buffer_bytes(rows, w.I, "mxfp8")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    # the weights are the bulk of each step's bytes: two copies (8 GB+ apart
    # would be needed to defeat the 256 MB cache; two sets already exceed it)
    nsets = args.sets or 2
    sets = []
    for i in range(nsets):
        w1, w1s = ep.pack_moe_weights(d(inp["w1_codes"]), d(inp["w1_scales"]), True)
        w2, w2s = ep.pack_moe_weights(d(inp["w2_codes"]), d(inp["w2_scales"]), False)
        sets.append(dict(
            x=d(inp["x"].view(np.int16)).view(torch.bfloat16), idx=d(inp["topk_idx"]), wt=d(inp["topk_weights"]),
            w1=w1, w1s=w1s, w2=w2, w2s=w2s,
            ws=torch.empty(ep.ep_workspace_bytes(w.T, w.k, w.E_local), dtype=torch.uint8, device=dev),
            rc=torch.empty(w.E_local, dtype=torch.int64, device=dev),
            recv=torch.empty(xb, dtype=torch.uint8, device=dev), a=torch.empty(ab, dtype=torch.uint8, device=dev),
            y=torch.empty(rows * w.H * 2, dtype=torch.uint8, device=dev),
            out=torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def phases(s):
        def lay():
            s["h"] = ep.ep_layout(s["idx"], w.E_local, w.T, s["rc"], s["ws"])

        def disp():
            ep.ep_dispatch(s["h"], s["x"], w.H, "mxfp8", s["recv"])

        def g1():
            ep.ep_moe_gmm1(s["h"], s["recv"], w.H, w.I, s["w1"], s["w1s"], "mxfp8", s["a"], recv_count=s["rc"])

        def g2():
            ep.ep_moe_gmm2(s["h"], s["a"], w.I, w.H, s["w2"], s["w2s"], s["y"], recv_count=s["rc"])

        def comb():
            ep.ep_combine(s["h"], s["y"], "none", w.H, s["idx"], s["wt"], s["out"])
        return [lay, disp, g1, g2, comb]

    runners = [phases(s) for s in sets]
    for i in range(max(args.warmup, nsets)):
        for f in runners[i % nsets]:
            f()
    torch.cuda.synchronize()
    R = int(sets[0]["rc"].sum().item())
    names = ["layout", "dispatch", "gmm1", "gmm2", "combine"]
    ms, ph_list, _, dist = timed_steps(runners, args.steps, stream)
    ph = dict(zip(names, ph_list))
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w.name, args.cpu_tokens or 256, moe=True)
    alg = moe_algorithmic(w, R)
    b, f = alg["bytes"], alg["flops"]
    gbps = lambda n: b[n] / (ph[n] * 1e-3) / 1e9
    tflops = lambda n: f[n] / (ph[n] * 1e-3) / 1e12
    roof = {"bound": "hbm", "kernel": "gmm1", "achieved": round(gbps("gmm1"), 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps("gmm1") / HBM_PEAK_GBPS, 4),
            "traffic": _traffic(w.name, MOE_TRAFFIC_FILE, MOE_KERNEL_SOURCES),
            "alg_bytes_per_launch": b["gmm1"], "avg_launch_ms": round(ph["gmm1"], 5),
            "mfma_tflops": round(tflops("gmm1"), 1),
            "mfma_frac": round(tflops("gmm1") / MFMA_FP8_PEAK_TFLOPS, 4)}
    print(json.dumps({
        "metric": "fused MoE step (dispatch, GMM1+SwiGLU+requant, GMM2, combine) tokens/s, H=7168 I=3072 k=6",
        "value": round(w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp8", "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} I={w.I} experts {w.E_local} of {w.E_total} k={w.k} "
                               f"MXFP8 activations and weights", "rows": R, "buffer_sets": nsets},
        "phase_ms": {n: round(v, 5) for n, v in ph.items()},
        "step_ms_phase_pass": dist,
        "phase_gbps": {n: round(gbps(n), 1) for n in names},
        "gemm_tflops": {n: round(tflops(n), 1) for n in ("gmm1", "gmm2")},
        "hbm_gbps": round(b["total"] / (ms * 1e-3) / 1e9, 1),
        "roofline": roof, "cpu_baseline": cpu}), flush=True)
    return 0


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries (HBM bytes per launch)
# ---------------------------------------------------------------------------

# kernels of each measured path: (label, substring of the kernel name)
PMC_KERNELS = {
    "path": [("combine", "combine_kernel"), ("dispatch", "dispatch_kernel"), ("layout_rank", "layout_rank_kernel"),
             ("layout_finalize", "layout_finalize_kernel"), ("layout_single", "layout_single_kernel")],
    "moe": [("gmm1", "mx_gmm_kernel<0>"), ("gmm2", "mx_gmm_kernel<2>"), ("dispatch", "dispatch_kernel"),
            ("combine", "combine_kernel")],
}


def _pmc_rows(path: str, counter: str) -> list:
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {path}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, moe: bool, copy_mib: int = 1024) -> dict:
    """HBM bytes per launch of the path's kernels from two rocprofv3 --pmc
    runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what
    the same counter reads for a device-to-device copy of `copy_mib` MiB in
    the same run (`--copy-probe-mib`), against the algorithmic bytes."""
    import numpy as np
    from combine_topk_idx_amd import workloads as W
    fetch, write = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0

    def calib(rows):
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise ValueError("no copy kernel in the counter run (run it with --copy-probe-mib)")
        return copies

    # the probe copy is the copy whose WRITE_SIZE is the copy's size; the
    # fetch run's copies come in the same order
    wcopies, fcopies = calib(write), calib(fetch)
    i = min(range(len(wcopies)), key=lambda j: abs(wcopies[j] - copy_kib))
    w_scale, f_scale = copy_kib / wcopies[i], copy_kib / fcopies[i]

    def per_launch(rows, sub):
        v = [float(r["Counter_Value"]) for r in rows if sub in r["Kernel_Name"]]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    if moe:
        w = W.MOE_WORKLOADS[workload]
        R = int((W.make_moe_inputs(w)["topk_idx"] >= 0).sum())
        alg = moe_algorithmic(w, R)["bytes"]
        measured, sources = "gmm1", MOE_KERNEL_SOURCES
    else:
        w = W.WORKLOADS[workload]
        idx = W.make_inputs(w)["topk_idx"]
        R = int(((idx >= 0) & (idx < w.E)).sum())
        alg = algorithmic_bytes(w, R)
        measured, sources = "combine", KERNEL_SOURCES
    kernels = {}
    for label, sub in PMC_KERNELS["moe" if moe else "path"]:
        fk, n = per_launch(fetch, sub)
        wk, _ = per_launch(write, sub)
        if fk is None:
            continue
        b = (fk * f_scale + wk * w_scale) * 1024.0
        a = alg.get(label)
        kernels[label] = {"launches": n, "fetch_kib_raw": round(fk, 3), "write_kib_raw": round(wk, 3),
                          "bytes": int(round(b)), "alg_bytes": a, "ratio": round(b / a, 4) if a else None}
    m = kernels[measured]
    return {"workload": workload, "kernel": measured, "source_hash": _source_hash(sources),
            "fetch_scale": f_scale, "write_scale": w_scale,
            "calibration": f"{copy_mib} MiB device-to-device copy read FETCH_SIZE {fcopies[i]:.0f} KiB and "
                           f"WRITE_SIZE {wcopies[i]:.0f} KiB",
            "bytes_per_launch": m["bytes"], "alg_bytes_per_launch": m["alg_bytes"],
            "traffic_over_alg": m["bytes"] / m["alg_bytes"], "kernels": kernels}


def _short_kernel_name(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def trace_summary(path: str, by_grid: bool = False) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats --output-format
    csv run: calls and average / min / max duration per kernel (from its
    *kernel_stats.csv), longest total first; with by_grid, per kernel and
    grid (workgroups x threads, from *kernel_trace.csv) with the median."""
    import csv
    import glob

    import numpy as np
    pattern = "*kernel_trace.csv" if by_grid else "*kernel_stats.csv"
    files = glob.glob(os.path.join(path, "**", pattern), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {pattern} under {path}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not by_grid:
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        out = ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in rows:
            out.append(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                       f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        return "\n".join(out)
    groups = {}
    for r in rows:
        wg = int(r["Workgroup_Size_X"])
        key = (_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(wg, 1), wg)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | workgroups x threads | calls | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(d)
        out.append(f"| `{key[0]}` | {key[1]} x {key[2]} | {a.size} | {a.mean():.2f} | {np.median(a):.2f} | "
                   f"{a.min():.2f} | {a.max():.2f} |")
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0: enough to exceed 1 GB)")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a known-size kernel "
                         "for calibrating rocprofv3 byte counters)")
    ap.add_argument("--combine-backward", default=None, metavar="QUANT",
                    help="time layout + ep_combine_backward (weighted reverse dispatch of a bf16 gradient "
                         "to the expert rows, quantised to QUANT, e.g. mxfp8) instead of the forward path")
    ap.add_argument("--row-align", type=int, default=1,
                    help="expert blocks start at multiples of this many rows (ep_layout_ex)")
    ap.add_argument("--expert-capacity", type=int, default=0,
                    help="every expert block has this many rows; later pairs are dropped (ep_layout_ex)")
    ap.add_argument("--interleaved", action="store_true",
                    help="receive rows hold their data then their scales (EP_RECV_INTERLEAVED)")
    ap.add_argument("--quant", default=None,
                    help="dispatch quantisation in place of the workload's own (e.g. fp8_b128_ue8m0)")
    ap.add_argument("--moe", default=None, metavar="WORKLOAD",
                    help="time the expert-MLP path (layout, MXFP8 dispatch, GMM1+SwiGLU+requant, GMM2, combine) "
                         "of a MoE workload, e.g. moe_share")
    ap.add_argument("--fused", action="store_true",
                    help="layout and dispatch through the one call ep_layout_dispatch (a single launch for compact "
                         "layouts of at most 2048 pairs)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as one captured HIP graph (no per-call host cost) instead of stream "
                         "launches")
    ap.add_argument("--probes", action="store_true",
                    help="time the probe kernels of libep_probe.so: launch floors at decode grids, combine's "
                         "gather and dispatch's scatter patterns at decode, the gather at the large size, 1 GiB "
                         "read / write / copy streams, the GEMMs' per-wave weight stream, the matrix-core rate")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="no GPU work: markdown table of a rocprofv3 --kernel-trace --stats csv run under DIR")
    ap.add_argument("--by-grid", action="store_true",
                    help="with --trace-summary: one row per kernel and grid, with the median")
    ap.add_argument("--pmc-summary", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench (with --copy-probe-mib) into HBM bytes per launch; prints JSON")
    ap.add_argument("--cpu-baseline-child", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-baseline-moe-child", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_baseline_child:
        cpu_baseline_child(args.cpu_baseline_child, args.cpu_tokens)
        return 0
    if args.cpu_baseline_moe_child:
        cpu_baseline_moe_child(args.cpu_baseline_moe_child, args.cpu_tokens)
        return 0
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.by_grid))
        return 0
    if args.pmc_summary:
        d = pmc_summary(*args.pmc_summary, args.moe or args.workload, bool(args.moe), args.copy_probe_mib or 1024)
        print(json.dumps(d, indent=1))
        return 0
    if args.probes:
        return probes_main(args)
    if args.combine_backward:
        return backward_main(args)
    if args.moe:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            return 2
        return moe_main(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"multi-GPU exchange)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from combine_topk_idx_amd import ep, workloads as W

    from dataclasses import replace
    w = W.WORKLOADS[args.workload]
    padded = args.row_align > 1 or args.expert_capacity > 0
    if padded:
        w = replace(w, row_align=args.row_align, expert_capacity=args.expert_capacity)
    variant = padded or args.interleaved or (args.quant is not None and args.quant != w.mode)
    if args.quant is not None:
        w = replace(w, mode=args.quant)
    if args.interleaved:
        w = replace(w, interleaved=True)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}: T={w.T} H={w.H} E={w.E} k={w.k} {w.mode} rows={w.max_rows}",
          file=sys.stderr, flush=True)
    inp = W.make_inputs(w)
    # padded blocks can hold far more rows than pairs: their bf16 N(0,1) expert
    # rows are drawn on the device (timing data only; parity is tested apart)
    y_host = W.make_expert_out(w) if w.combine_input == "normal" and not padded else None
    y_dev = w.combine_input == "normal" and padded

    total_recv, _ = ep.ep_buffer_bytes(w.max_rows, w.H, w.mode, w.interleaved)
    per_set = (w.T * w.H * 2 * 2 + total_recv + (w.max_rows * w.H * 2 if w.combine_input == "normal" else 0))
    nsets = args.sets or max(2, -(-(1 << 30) // max(per_set, 1)))
    nsets = min(nsets, 64)

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    sets = []
    for i in range(nsets):
        s = {
            "x": dev_bf16(inp["x"]),
            "idx": torch.from_numpy(inp["topk_idx"]).to(dev),
            "w": torch.from_numpy(inp["topk_weights"]).to(dev),
            "ws": torch.empty(ep.ep_workspace_bytes_ex(w.t_max, w.k, w.E, w.row_align, w.expert_capacity),
                              dtype=torch.uint8, device=dev),
            "rc": torch.empty(w.E, dtype=torch.int64, device=dev),
            "recv": torch.empty(total_recv, dtype=torch.uint8, device=dev),
            "out": torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev),
        }
        if y_host is not None:
            s["y"] = dev_bf16(y_host).view(torch.uint8).reshape(-1) if i == 0 else sets[0]["y"].clone()
        elif y_dev and i == 0:
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed)
            y = torch.empty((w.max_rows, w.H), dtype=torch.bfloat16, device=dev)
            for r0 in range(0, w.max_rows, 16384):
                n = min(16384, w.max_rows - r0)
                y[r0:r0 + n] = torch.randn((n, w.H), generator=g, device=dev).to(torch.bfloat16)
            s["y"] = y.view(torch.uint8).reshape(-1)
        elif y_dev:
            s["y"] = sets[0]["y"].clone()
        sets.append(s)
    del y_host
    stream = torch.cuda.current_stream()
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def phases(s):
        """The three calls of one step on buffer set s, on torch's current stream."""
        def lay():
            if padded:
                s["h"] = ep.ep_layout_ex(s["idx"], w.E, w.t_max, w.row_align, w.expert_capacity, s["rc"], s["ws"])
            else:
                s["h"] = ep.ep_layout(s["idx"], w.E, w.t_max, s["rc"], s["ws"])

        def disp():
            ep.ep_dispatch(s["h"], s["x"], w.H, w.mode, s["recv"], interleaved=w.interleaved)

        def lay_disp():
            s["h"] = ep.ep_layout_dispatch(s["idx"], w.E, w.t_max, s["rc"], s["ws"], s["x"], w.H, w.mode, s["recv"],
                                           row_align=w.row_align, expert_capacity=w.expert_capacity,
                                           interleaved=w.interleaved)

        def comb():
            if w.combine_input == "identity":
                ep.ep_combine(s["h"], s["recv"], w.mode, w.H, s["idx"], s["w"], s["out"], interleaved=w.interleaved)
            elif w.combine_input == "scaled_dispatch":
                # the x1.5 expert step is not part of the path: combine reads
                # the dispatched bf16 rows (same bytes, same work)
                ep.ep_combine(s["h"], s["recv"], "none", w.H, s["idx"], s["w"], s["out"])
            else:
                ep.ep_combine(s["h"], s["y"], "none", w.H, s["idx"], s["w"], s["out"])
        return [lay_disp, comb] if args.fused else [lay, disp, comb]

    runners = [phases(s) for s in sets]
    print(f"[bench] {nsets} buffer sets, warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for i in range(max(args.warmup, nsets)):
        for f in runners[i % nsets]:
            f()
    torch.cuda.synchronize()
    R = int(sets[0]["rc"].sum().item())
    # timed region: the throughput pass of timed_steps, on the launch stream;
    # the per-phase times (and combine's launch time) come from its phase pass
    ms_per_step, ph, wall_s, dist = timed_steps(runners, args.steps, stream)
    lay_ms, disp_ms, comb_ms = (ph[0], None, ph[1]) if args.fused else ph
    stream_ms = ms_per_step
    if args.graph:
        # the timed steps as one graph replay; the phases stay those of the
        # stream pass
        ms_per_step = graph_steps(runners, args.steps, stream)

    b = algorithmic_bytes(w, R)
    gbps = b["total"] / (ms_per_step * 1e-3) / 1e9
    comb_gbps = b["combine"] / (comb_ms * 1e-3) / 1e9
    traffic = None if variant else _traffic(w.name)
    roof = {"bound": "hbm", "kernel": "combine", "achieved": round(comb_gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(comb_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "alg_bytes_per_launch": b["combine"], "avg_launch_ms": round(comb_ms, 5)}

    warm_ms = None
    if nsets > 2:
        # the same steps on one buffer set, whose inputs then stay in the
        # 256 MB last-level cache: reported beside the cold figure, labelled,
        # never as the metric
        warm_ms = timed_steps([runners[0]], args.steps, stream)[0]

    cpu = None
    if not args.no_cpu_baseline and not variant:
        # one 1024-token chunk of the large workloads (about 5 s per run of
        # the oracle; three runs keep the default bench within minutes)
        tokens = args.cpu_tokens or {"large": 1024, "prefill": 1024}.get(w.name, w.T)
        print(f"[bench] cpu oracle on {tokens} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w.name, tokens)

    line = {
        "metric": METRIC, "value": round(w.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} k={w.k} ids={w.idx_dtype} "
                               f"dispatch={w.mode} routing={w.routing} unrouted={w.neg_frac} "
                               f"combine_input={w.combine_input}",
                   "T": w.T, "H": w.H, "E": w.E, "k": w.k, "rows": R, "buffer_sets": nsets,
                   "row_align": w.row_align, "expert_capacity": w.expert_capacity, "interleaved": w.interleaved,
                   "receive_rows": w.max_rows, "launch": "graph" if args.graph else "stream",
                   "layout_dispatch": "one call (ep_layout_dispatch)" if args.fused else "two calls"},
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": b["total"],
        "phase_ms": ({"layout_dispatch": round(lay_ms, 5), "combine": round(comb_ms, 5)} if args.fused else
                     {"layout": round(lay_ms, 5), "dispatch": round(disp_ms, 5), "combine": round(comb_ms, 5)}),
        "phase_gbps": ({"combine": round(comb_gbps, 1)} if args.fused else
                       {"dispatch": round(b["dispatch"] / (disp_ms * 1e-3) / 1e9, 1), "combine": round(comb_gbps, 1)}),
        "wall_s": round(wall_s, 4),
        "step_ms_phase_pass": dist,
        "stream_ms_per_step": round(stream_ms, 5),
        "warm_one_set_ms_per_step": None if warm_ms is None else round(warm_ms, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
