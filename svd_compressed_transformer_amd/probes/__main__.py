"""Build and run the measurement probes:

    python -m svd_compressed_transformer_amd.probes [grid_barrier] [phase_boundary]

grid_barrier: the cost of one grid-wide barrier with one workgroup per CU (see grid_barrier.hip);
prints one JSON line per (mode, workgroup count).
phase_boundary: a decode layer-step modelled as 10 dependent streaming phases, as 10 kernels in a
graph against one persistent kernel with grid barriers, with and without prefetching the next
phase's first loads before each barrier; then the 9 phases left with the attention merge inside
the attention kernel, at the decode kernels' grids and at 512, 1024 and 2048 workgroups a phase,
with 25 / 50 / 100% of each next phase prefetched into the Infinity Cache, and with each
projection's two phases in one launch on separate workgroups (see phase_boundary.hip); one JSON
line per variant.
"""
from __future__ import annotations

import os
import subprocess
import sys

from svd_compressed_transformer_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("grid_barrier", "phase_boundary")


def binary(name: str) -> str:
    return os.path.join(_build.BUILD_DIR, f"probe_{name}")


def build(name: str) -> str:
    os.makedirs(_build.BUILD_DIR, exist_ok=True)
    out = binary(name)
    cmd = [_build.HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(HERE, f"{name}.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for probe {name}:\n{r.stderr}")
    return out


def main(argv) -> int:
    names = argv or list(PROBES)
    for n in names:
        if n not in PROBES:
            raise SystemExit(f"unknown probe {n!r}; known: {PROBES}")
        exe = binary(n) if os.path.exists(binary(n)) else build(n)
        r = subprocess.run([exe])
        if r.returncode != 0:
            return r.returncode
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
