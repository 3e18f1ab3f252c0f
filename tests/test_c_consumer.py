"""The library used from plain C: tests/c_abi/ep_consumer.c includes only
include/ep.h (and the HIP runtime API for its own buffers), is compiled as
strict C99 by gcc and linked to the in-tree libep.so by the library build.

Without a GPU it runs the host-only calls (size queries, a check that fails
before launching, the last-error text); on the GPU it runs one layout ->
dispatch -> combine round trip and checks the counts against the expert
histogram and combine(dispatch(x)) against the closed form k_eff * x for
unit weights and unquantised rows ("Low-Latency Mode API",
low_latency_dispatch / low_latency_combine)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "c_abi", "ep_consumer")
SRC = PROG + ".c"


def _run(mode: str) -> str:
    assert os.path.exists(PROG), "tests/c_abi/ep_consumer is missing: run the library build"
    assert os.path.getmtime(PROG) >= os.path.getmtime(SRC), "tests/c_abi/ep_consumer is older than its source"
    print(f"\n[case] C consumer {mode}", flush=True)
    sys.stdout.flush()
    r = subprocess.run([PROG, mode], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    return r.stdout


def test_c_consumer_host():
    out = _run("host")
    assert "FAIL" not in out


@pytest.mark.gpu
def test_c_consumer_gpu_round_trip():
    out = _run("gpu")
    assert "combine(dispatch(x)) == k_eff * x for every token" in out
