"""Build libcorrector.so (gfx950) in-tree with hipcc.

Run ``python -m draft_correction_amd.build`` or call ``build()``.  The shared
library lands next to this file so it travels with the source tree.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcorrector.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-fPIC", "-shared", "-std=c++17", "--offload-arch=" + ARCH,
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libcorrector.so``; return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc"] + FLAGS + ["-o", tmp] + sources()
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
