"""Build the HIP library ``libnvfp4.so`` for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` and the
objects are linked into ``nvfp4_w4a4_quantized_02_amd/libnvfp4.so``; the
benchmark's reference kernels (``probe/*.hip``) go into ``libnvfp4_probe.so``.  Run as
``python nvfp4_w4a4_quantized_02_amd/build.py`` (a script: importing the
package itself needs the built library).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
PROBE = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libnvfp4_probe.so")
ARCH = "gfx950"

# -ffp-contract=off keeps every fp32 step of the quantizer a separately
# rounded operation; IEEE division and subnormals stay on (the defaults).
# Packed fp32 instructions are switched off for the device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libnvfp4.so and the benchmark's reference-kernel library
    libnvfp4_probe.so (a plain HBM read, not part of the NVFP4 path)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBE, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
