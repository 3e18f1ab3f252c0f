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
BUILD = os.path.join(HERE, "_build")
SOURCES = ["layout.hip", "dispatch.hip", "combine.hip", "moe.hip", "ep_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, build_dir: str, defines: tuple) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile every source and link the library (default: libep.so next to
    this file; ``defines`` are extra -D macros, e.g. launch-shape overrides
    from csrc/tuning.hpp); returns the library path."""
    build_dir = BUILD if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(defines)), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
