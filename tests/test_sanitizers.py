"""CPU runs of the oracle and of the C ABI's validation path under the
address and undefined-behaviour sanitizers.

* The oracle (plain C) is built with gcc and driven over ragged shapes,
  bf16 and fp32 inputs and zero tensors (tests/sanitize/oracle_driver.c).
* The ABI layer (csrc/capi.hip) is built with its host code instrumented
  (the device code is not) and linked against launchers that abort
  (tests/sanitize/launch_stubs.hip): every call of tests/sanitize/abi_driver.c
  must be rejected, or accepted as empty, on the host, and every workspace
  size must be computed without overflow for every extreme shape.

A sanitizer finding aborts the driver, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "nvfp4_w4a4_quantized_02_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"

# host-side sanitizers on hipcc lines: each option behind -Xarch_host
HIPCC_HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp", os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr


def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    if not (os.path.exists(hipcc) and os.path.exists(os.path.join(LLVM, "clang++"))):
        pytest.skip("hipcc / ROCm clang not available")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             *HIPCC_HOST_SAN]
    capi, stubs = str(tmp_path / "capi.o"), str(tmp_path / "stubs.o")
    _run([hipcc, *flags, "-c", os.path.join(CSRC, "capi.hip"), "-o", capi])
    _run([hipcc, *flags, "-c", os.path.join(SAN, "launch_stubs.hip"), "-o", stubs])
    drv, exe = str(tmp_path / "driver.o"), str(tmp_path / "abi_san")
    _run([os.path.join(LLVM, "clang"), "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    _run([os.path.join(LLVM, "clang++"), "-fsanitize=address,undefined", drv, capi, stubs, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations outlive main, so leak checking is off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr
