"""Build libzdo.so (the HIP library behind include/zdo.h) in-tree for gfx950.

    python -m zero_distributed_optimizer_amd.build

Flags: -ffp-contract=off (no FMA contraction: the step's fp32 operations are
rounded one by one), HIP's default IEEE division and square root, and the
packed-fp32 instructions turned off.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzdo.so")
# A test build whose launches are capped at 64 workgroups, so that every
# kernel walks its tiles through the grid-stride continuation (in the real
# build only launches of more than 2^24 tiles do).
GRID_LOOP_LIB = os.path.join(HERE, "libzdo_gridloop.so")
GRID_LOOP_FLAGS = ["-DZDO_MAX_GRID=64"]
SOURCES = ["plan.cpp", "abi.cpp", "kernels.hip"]
HEADERS = ["zdo_internal.h", "kernels.h"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-parameter", "-Wl,--no-undefined",
]


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(CSRC, h) for h in HEADERS] + \
        [os.path.join(INCLUDE, "zdo.h")]


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    out = out or LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("libzdo build failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    """The library and its grid-loop test build, compiled side by side."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        jobs = [ex.submit(build, verbose), ex.submit(build, verbose, GRID_LOOP_FLAGS, GRID_LOOP_LIB)]
        return [j.result() for j in jobs]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
