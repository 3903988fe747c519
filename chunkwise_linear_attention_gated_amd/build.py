"""Build the HIP library ``_harts.so`` in-tree for gfx950 (hipcc).

Sources: ``csrc/host/*.cpp`` (C++17 planner), ``csrc/abi.cpp`` (C ABI),
``csrc/kernels/*.hip`` (device code).  Every call rebuilds; objects go to
``_build/`` next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "_harts.so")
ARCH = os.environ.get("HARTS_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc")]
# device code: no packed-fp32 instructions (they are not used on this target)
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-core accumulators in VGPRs: avoids accumulator shuffles across loop iterations
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src: str, obj: str, device: bool) -> str:
    cmd = [HIPCC] + COMMON + (DEVICE + ["-x", "hip"] if device else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    for src in sorted(glob.glob(os.path.join(HERE, "csrc", "host", "*.cpp"))) + [os.path.join(HERE, "csrc", "abi.cpp")]:
        jobs.append((src, os.path.join(bdir, os.path.basename(src) + ".o"), False))
    for src in sorted(glob.glob(os.path.join(HERE, "csrc", "kernels", "*.hip"))):
        jobs.append((src, os.path.join(bdir, os.path.basename(src) + ".o"), True))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, SO)
    if verbose:
        print("built", SO)
    return SO


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
