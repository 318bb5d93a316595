"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

gba_api.hip (the C ABI: argument checks, schedule choice, the on-disk schedule
cache and its file locking) is compiled again with both sanitizers on its host
side only (-Xarch_host; the device code is built as usual and never runs
here), linked with the other objects of the current build and with
tests/host_sanitize_check.c, and run without a GPU. The program covers every
GPU-less path: argument errors of each entry point, the schedule table, and the
cache with missing, corrupt, truncated and oversized files, an unwritable
directory, GBA_DISABLE_CACHE and writers in several threads. Any sanitizer
report (heap or stack overflow, use after free, leak, undefined behaviour)
aborts the run and fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_dense_gemm_bias_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer", "-g"]


def _objects():
    """The current build's objects other than the C ABI's (build.py names each
    after its source)."""
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o")
            for s in sorted(glob.glob(os.path.join(CSRC, "*.hip")))
            if os.path.basename(s) != "gba_api.hip"]
    return objs


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    for tool in (HIPCC, CLANG, CLANGXX):
        if not os.path.exists(tool):
            pytest.skip("ROCm compilers not installed")
    objs = _objects()
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.skip("library not built (run build() first): %s" % missing[0])
    d = str(tmp_path_factory.mktemp("san"))
    api = os.path.join(d, "gba_api_san.o")
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    cmd = ([HIPCC, "-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", '-DGBA_BUILD_ID="sanitize"']
           + host_san + ["-c", os.path.join(CSRC, "gba_api.hip"), "-o", api])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # The host objects really are instrumented.
    syms = subprocess.run(["nm", api], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    prog_o = os.path.join(d, "check.o")
    r = subprocess.run([CLANG, "-O1", "-I" + os.path.join(ROOT, "include")] + SAN +
                       ["-c", os.path.join(ROOT, "tests", "host_sanitize_check.c"), "-o", prog_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = os.path.join(d, "host_sanitize_check")
    r = subprocess.run([CLANGXX, "-fsanitize=address", "-fsanitize=undefined", prog_o, api] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread",
                        "-lm", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe, d


def test_host_code_is_clean_under_asan_and_ubsan(program):
    exe, d = program
    scratch = os.path.join(d, "scratch")
    shutil.rmtree(scratch, ignore_errors=True)
    os.makedirs(scratch)
    env = dict(os.environ)
    env.pop("GBA_DISABLE_CACHE", None)
    env.update(ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, scratch], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report and "LeakSanitizer" not in report, report[-6000:]
    assert "runtime error" not in report, report[-6000:]
    assert r.returncode == 0 and "host sanitize check ok" in r.stdout, report[-6000:]
    # every writer thread's entries reached the shared cache file
    with open(os.path.join(scratch, "threads", "schedules.json")) as f:
        assert len(f.read().splitlines()) == 2 + 8 * 24
