"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The corrector library is rebuilt with its host code instrumented (device
  code is unchanged: every sanitizer flag is given to the host pass only) and
  a C driver runs the ABI's host paths through it: descriptor validation,
  argument checks, n_req = 0 no-ops and the handle life cycle (calls and a
  second destroy on a destroyed handle).  Every call it makes fails host
  validation or is a no-op, so nothing is launched; the child also sees no
  GPU (HIP_VISIBLE_DEVICES=-1), so a call that wrongly passed validation
  would fail to launch rather than touch a device.
* The oracle is rebuilt with gcc's sanitizers and driven over every entry
  point on small seeded inputs in a child interpreter.

Either run fails on the first sanitizer report.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HERE = os.path.dirname(os.path.abspath(__file__))

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _env(**extra):
    env = dict(os.environ)
    env.update(extra)
    return env


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_abi_host_code_under_asan_ubsan():
    from draft_correction_amd import build as hipbuild
    os.makedirs(OUT, exist_ok=True)
    lib = hipbuild.build(extra_flags=tuple(HOST_SAN), lib=os.path.join(OUT, "libcorrector.so"),
                         obj_dir=os.path.join(OUT, "obj"))
    exe = os.path.join(OUT, "abi_host_check")
    clang = "/opt/rocm/llvm/bin/clang"
    subprocess.check_call([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", exe, os.path.join(HERE, "sanitize", "abi_host_check.c"),
                           lib, "-Wl,-rpath," + OUT])
    # leak checking is off: the HIP runtime keeps process-lifetime allocations
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=_env(HIP_VISIBLE_DEVICES="-1",
                                  ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
                                  UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi host checks passed" in res.stdout


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    res = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "oracle_drive.py")],
                         capture_output=True, text=True, timeout=600,
                         env=_env(LD_PRELOAD=asan, DRAFT_ORACLE_LIB=lib, OMP_NUM_THREADS="2",
                                  ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                                  UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "oracle driven under sanitizers" in res.stdout
