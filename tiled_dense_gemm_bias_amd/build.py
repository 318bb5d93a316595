"""Build libgba.so (the gfx950 HIP library) in-tree.

    python -m tiled_dense_gemm_bias_amd.build [--isa]

Each csrc/*.hip file is compiled on its own (in parallel) with hipcc for
gfx950 only, then linked into tiled_dense_gemm_bias_amd/libgba.so. --isa also
keeps the gfx950 assembly of every file under _build/isa/ for inspection
(MFMA / LDS / spill checks).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgba.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I" + INCLUDE, "-I" + CSRC,
    # No packed-fp32 VALU instructions in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build_id() -> str:
    """Hash of everything the kernels are compiled from (sources, the public
    header, the flags): part of every schedule-cache key, so that a schedule
    tuned on other kernels is never reused."""
    h = hashlib.sha256()
    for fn in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                     + [os.path.join(INCLUDE, "gba.h")]):
        h.update(os.path.basename(fn).encode())
        with open(fn, "rb") as f:
            h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]


def _compile(src: str, isa: bool, bid: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    if os.path.basename(src) == "gba_api.hip":
        cmd.append('-DGBA_BUILD_ID="%s"' % bid)
    if isa:
        isadir = os.path.join(BUILD, "isa")
        os.makedirs(isadir, exist_ok=True)
        cmd += ["-save-temps=obj"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, res.stderr))
    if isa:
        base = os.path.join(BUILD, os.path.basename(src)[:-4])
        for s in glob.glob(base + "-hip-amdgcn-amd-amdhsa-" + ARCH + ".s"):
            shutil.copy(s, os.path.join(BUILD, "isa", os.path.basename(s)))
    return obj


def build(isa: bool = False, jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    bid = build_id()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, isa, bid), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    res = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs,
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--isa", action="store_true", help="keep gfx950 assembly under _build/isa")
    ap.add_argument("-j", "--jobs", type=int, default=0)
    a = ap.parse_args(argv)
    print(build(isa=a.isa, jobs=a.jobs))
    return 0


if __name__ == "__main__":
    sys.exit(main())
