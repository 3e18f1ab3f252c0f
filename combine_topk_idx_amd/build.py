"""Build libep.so (HIP, gfx950) in-tree with hipcc.

    python -m combine_topk_idx_amd.build

Flags that matter for results:
  -ffp-contract=off                      no fused multiply-add: combine's
                                         multiply and add are rounded separately
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE float32 division for the
                                         quantisation multipliers and scales
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         keep the compiler from emitting packed
                                         fp32 instructions
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libep.so")
PROBE_LIB = os.path.join(HERE, "libep_probe.so")   # measurement probes of bench.py --probes
PROBE_SOURCES = ["probes.hip"]
BUILD = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)
# a plain C99 program that uses the library only through include/ep.h
CONSUMER_SRC = os.path.join(ROOT, "tests", "c_abi", "ep_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "c_abi", "ep_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = ["layout.hip", "dispatch.hip", "combine.hip", "moe.hip", "static_ws.hip", "ep_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# AddressSanitizer for the host code only (the device code cannot carry it
# here): each -fsanitize= goes to the host pass alone
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str, defines: tuple, extra: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *extra, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, out: str, extra: tuple = ()) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build_consumer() -> str:
    """Compiles tests/c_abi/ep_consumer.c with gcc as strict C99 against
    include/ep.h (the HIP headers as system headers) and links it to the
    in-tree libep.so, found at run time relative to the program."""
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), CONSUMER_SRC,
           "-L", HERE, "-lep", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_topk_idx_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", CONSUMER + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on the C consumer:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(CONSUMER + ".tmp", CONSUMER)
    return CONSUMER


def build(verbose: bool = False, out: str = LIB, defines: tuple = (), host_asan: bool = False) -> str:
    """Compile every source and link the library (default: libep.so next to
    this file; ``defines`` are extra -D macros, e.g. launch-shape overrides
    from csrc/tuning.hpp); returns the library path.  The default build also
    links the measurement probes of ``bench.py --probes`` (libep_probe.so)
    and the plain C user of the header, tests/c_abi/ep_consumer.

    host_asan: the host code (argument checks, handles, launch set-up) with
    AddressSanitizer, for the host-only ABI tests on a machine without a
    GPU; load it with the ASan runtime preloaded (the runtime's path is
    ``hipcc -print-file-name=libclang_rt.asan-x86_64.so``) and
    ASAN_OPTIONS=detect_leaks=0, and build again without it afterwards."""
    build_dir = (BUILD if out == LIB else out + ".build") + ("_asan" if host_asan else "")
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if out == LIB else [])
    cflags = tuple(HOST_ASAN) if host_asan else ()
    lflags = ("-Xarch_host", "-fsanitize=address", "-shared-libasan") if host_asan else ()
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, build_dir, tuple(defines), cflags), srcs)))
    _link([objs[s] for s in SOURCES], out, lflags)
    if out == LIB:
        _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, lflags)
        if not host_asan:
            build_consumer()
    if verbose:
        print(f"built {out}" + (f" and {PROBE_LIB}" if out == LIB else "") + (" (host ASan)" if host_asan else ""))
    return out


if __name__ == "__main__":
    build(verbose=True, host_asan="--host-asan" in sys.argv[1:])
    sys.exit(0)
