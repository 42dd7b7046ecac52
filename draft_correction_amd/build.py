"""Build libcorrector.so (gfx950) in-tree with hipcc.

Run ``python -m draft_correction_amd.build`` or call ``build()``.  Each HIP
source is compiled to an object of its own (in parallel, under ``_build/``)
and the objects are linked into the shared library, which lands next to this
file so it travels with the source tree.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcorrector.so")
OBJ = os.path.join(os.path.dirname(HERE), "_build", "corrector")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-fPIC", "-std=c++17", "--offload-arch=" + ARCH,
    # never emit packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "packed-fp32-ops' is not a recognized feature"


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list) -> tuple:
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    return res.returncode, msgs


def build(verbose: bool = False, extra_flags: tuple = (), lib: str = LIB, obj_dir: str = OBJ) -> str:
    """Compile every HIP source and link ``libcorrector.so``; return its path.
    ``extra_flags`` are appended to every compile and link line (a sanitizer
    build of the host code passes its flags here, with ``lib`` and
    ``obj_dir`` pointing elsewhere)."""
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
    jobs = [["hipcc"] + FLAGS + list(extra_flags) + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        results = list(ex.map(_run, jobs))
    msgs = []
    for (rc, m), s in zip(results, srcs):
        msgs += m
        if rc != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (s, "\n".join(m)))
    tmp = lib + ".tmp%d" % os.getpid()
    rc, m = _run(["hipcc", "-shared", "-fPIC", "--hip-link", "--offload-arch=" + ARCH] + list(extra_flags)
                 + ["-o", tmp] + objs)
    msgs += m
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(m))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
