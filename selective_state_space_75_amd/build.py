"""Build libmamba_scan.so (HIP, gfx950) in-tree with hipcc.

    python -m selective_state_space_75_amd.build

Every .hip file under csrc/ is compiled to an object (in parallel), and the
objects are linked into one shared library that exports the C ABI of
include/mamba_scan.h.  Packed-FP32 instructions are disabled for the device
code (the host pass warns that it does not know the feature; harmless).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmamba_scan.so")
ARCH = os.environ.get("MAMBA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]
# Per-file additions.  ssd.hip: MFMA accumulators in ordinary VGPRs, so the
# state the SSD kernels update with both MFMA and VALU instructions is not
# copied between AGPRs and VGPRs every chunk.
FILE_FLAGS = {"ssd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d): %s\n%s" % (res.returncode, " ".join(cmd), err))
    return err


def build(verbose: bool = False) -> str:
    incs = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="mamba_build_")
    try:
        jobs = []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            extra = FILE_FLAGS.get(os.path.basename(src), [])
            jobs.append(([HIPCC] + FLAGS + extra + incs + ["-c", "-o", obj, src], obj))
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            futs = []
            for cmd, _ in jobs:
                if verbose:
                    print(" ".join(cmd), flush=True)
                futs.append(ex.submit(_run, cmd))
            for f in futs:
                err = f.result()
                if err.strip() and verbose:
                    print(err, file=sys.stderr)
        tmp = LIB + ".tmp%d" % os.getpid()
        link = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
