"""No kernel of the library uses scratch (private) memory.

A kernel with a private segment pays for it at every launch, and register
spills or an outlined device call (which takes the caller's live state
through the stack) show up there first.  Each kernel source is compiled for
gfx950 with the compiler's resource-usage remarks and every kernel must
report zero scratch bytes per lane.  Runs on the CPU (hipcc cross-compiles).
"""
import concurrent.futures as cf
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "nvfp4_w4a4_quantized_02_amd")


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("nvfp4_hip_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _remarks(src, tmp):
    b = _build_module()
    out = os.path.join(tmp, os.path.basename(src) + ".dev.o")
    cmd = [b.hipcc(), *b.HIPCC_FLAGS, "--cuda-device-only", "-c", src, "-o", out,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stderr[-3000:])
    return r.stderr


def _kernels(remarks):
    """[(kernel name, scratch bytes per lane)] from the remarks of one file."""
    names = re.findall(r"remark: Function Name: (\S+)", remarks)
    scratch = [int(v) for v in re.findall(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    assert len(names) == len(scratch), "unexpected remark format"
    return list(zip(names, scratch))


def test_no_kernel_uses_scratch(tmp_path):
    try:
        _build_module().hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        remarks = list(ex.map(lambda s: _remarks(s, str(tmp_path)), srcs))
    seen, bad = 0, []
    for src, rem in zip(srcs, remarks):
        for name, scratch in _kernels(rem):
            seen += 1
            if scratch:
                bad.append("%s: %s uses %d bytes of scratch per lane" % (os.path.basename(src), name, scratch))
    assert seen >= 20, "found only %d kernels" % seen
    assert not bad, "\n".join(bad)
