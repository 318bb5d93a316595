"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function include/gba.h declares, and
reject bad arguments synchronously, before touching a device. With no GPU (as
in a CPU-only container) a well-formed call must fail with GBA_ERR_DEVICE
rather than crash.
"""
import ctypes
import subprocess
import sys

import pytest

import tiled_dense_gemm_bias_amd as gba

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ACT, ERR_ALIGN, ERR_ALIAS, ERR_DEVICE = range(8)
ERR_SCHEDULE = 9

P16 = 0x10000      # a 16-byte-aligned fake address: never dereferenced by these calls


def _gpu_present():
    # Count devices in a child process so this process never initialises HIP.
    code = "import torch; print(torch.cuda.device_count())"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    try:
        return int(out.stdout.strip().splitlines()[-1]) > 0
    except (ValueError, IndexError):
        return False


@pytest.fixture(scope="module")
def lib():
    return gba.lib()


def test_library_exports_every_declared_function(lib):
    names = gba.header_functions()
    for n in ("gemm_bias_act", "gemm", "bias_act", "gba_set_stream", "gba_set_schedule",
              "gba_get_schedule", "gba_autotune", "gba_status_string", "gba_version"):
        assert n in names
    cdll = ctypes.CDLL(gba.LIB_PATH)
    missing = [n for n in names if not hasattr(cdll, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert gba.version().count(".") == 2
    for s in range(11):
        assert lib.gba_status_string(s)
    assert b"unknown" in lib.gba_status_string(99)


def test_schedule_table(lib):
    scheds = gba.list_schedules()
    assert len(scheds) == lib.gba_num_schedules() >= 4
    for s in scheds:
        # the pages' shared-memory filter, against the 160 KiB LDS of a CU
        assert (s["bm"] * s["bk"] + s["bk"] * s["bn"]) * 2 * s["stages"] <= 160 * 1024
        # whole MFMA blocks per wave: 16x16 (kernels 3, 4), else 32x32
        blk = 16 if s["kernel"] in (3, 4) else 32
        assert s["bm"] % (blk * s["wm"]) == 0 and s["bn"] % (blk * s["wn"]) == 0
    assert any((s["bm"], s["bn"], s["bk"]) == (128, 128, 32) for s in scheds)
    assert lib.gba_list_schedule(len(scheds), ctypes.byref(gba.Schedule())) == ERR_SCHEDULE


def test_set_schedule_validation(lib):
    good = gba.list_schedules()[0]
    gba.set_schedule(good)
    gba.set_schedule(None)
    with pytest.raises(gba.GbaError):
        gba.set_schedule(dict(good, bm=96))
    with pytest.raises(gba.GbaError):
        gba.set_schedule(dict(good, raster=3))
    with pytest.raises(gba.GbaError):
        gba.set_schedule(dict(good, group_m=0))


def call(lib, A=P16, B=P16, bias=None, C=P16 * 64, M=64, N=64, K=64, act=0, dt=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gemm_bias_act(v(A), v(B), v(bias), v(C), M, N, K, act, dt)


def test_argument_errors_are_synchronous_and_precede_device_use(lib):
    assert call(lib, dt=2) == ERR_DTYPE
    assert call(lib, act=6) == ERR_ACT
    assert call(lib, act=-1) == ERR_ACT
    assert call(lib, M=-1) == ERR_SHAPE
    assert call(lib, K=1 << 24) == ERR_SHAPE
    assert call(lib, C=None) == ERR_NULL
    assert call(lib, A=None) == ERR_NULL
    assert call(lib, K=12) == ERR_ALIGN
    assert call(lib, N=60) == ERR_ALIGN
    assert call(lib, A=P16 + 2) == ERR_ALIGN
    assert call(lib, bias=P16 * 200 + 8) == ERR_ALIGN
    assert call(lib, C=P16 + 64) == ERR_ALIAS            # C overlaps A
    assert call(lib, bias=P16 * 64 + 128) == ERR_ALIAS   # C overlaps bias
    # nothing to do: no device needed, no launch
    assert call(lib, M=0) == OK
    assert call(lib, N=0, A=None, B=None) == OK


def call8(lib, A=P16, W=P16, bias=None, C=P16 * 64, M=64, N=64, K=64, scale=1.0, act=0, fmt=0,
          dt=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.gemm_bias_act_fp8_nt(v(A), v(W), v(bias), v(C), M, N, K, scale, act, fmt, dt)


def test_fp8_argument_errors_precede_device_use(lib):
    assert call8(lib, fmt=2) == ERR_DTYPE
    assert call8(lib, dt=2) == ERR_DTYPE
    assert call8(lib, act=6) == ERR_ACT
    assert call8(lib, M=-1) == ERR_SHAPE
    assert call8(lib, scale=float("inf")) == ERR_SHAPE
    assert call8(lib, scale=float("nan")) == ERR_SHAPE
    assert call8(lib, C=None) == ERR_NULL
    assert call8(lib, W=None) == ERR_NULL
    assert call8(lib, K=24) == ERR_ALIGN     # 8-bit rows must be whole 16-byte chunks
    assert call8(lib, N=60) == ERR_ALIGN
    assert call8(lib, A=P16 + 8) == ERR_ALIGN
    assert call8(lib, C=P16 + 32) == ERR_ALIAS
    assert call8(lib, M=0) == OK
    assert call8(lib, N=0, A=None, W=None) == OK


def test_ex_and_workspace_argument_errors_precede_device_use(lib):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    ex = lambda flags=0, ws=None, nb=0, **kw: lib.gemm_bias_act_ex(
        v(P16), v(P16), None, v(P16 * 64), 64, 64, 64, kw.get("act", 0), kw.get("dt", 0), flags,
        v(ws), nb)
    assert ex(flags=2) == ERR_SHAPE              # unknown flag bit
    assert ex(act=6) == ERR_ACT
    assert ex(ws=P16 * 200 + 8, nb=1 << 20) == ERR_ALIGN
    assert ex(ws=P16 * 64 + 256, nb=1 << 20) == ERR_ALIAS   # overlaps C
    size = ctypes.c_size_t(123)
    assert lib.gba_workspace_size(64, 64, 64, 0, 0, 8, ctypes.byref(size)) == ERR_SHAPE
    assert lib.gba_workspace_size(-1, 64, 64, 0, 0, 0, ctypes.byref(size)) == ERR_SHAPE
    assert lib.gba_workspace_size(0, 64, 64, 0, 0, 0, ctypes.byref(size)) == OK and size.value == 0
    assert lib.gba_workspace_size(64, 64, 64, 0, 0, 0, None) == ERR_NULL
    sch, splits = gba.Schedule(), ctypes.c_int(7)
    assert lib.gba_split_plan(64, 64, 64, 0, 0, 0, None, ctypes.byref(splits)) == ERR_NULL
    assert lib.gba_split_plan(64, 64, 64, 0, 0, 0, ctypes.byref(sch), None) == ERR_NULL
    assert lib.gba_split_plan(64, 64, 64, 0, 0, 2, ctypes.byref(sch), ctypes.byref(splits)) == ERR_SHAPE
    assert lib.gba_split_plan(64, -1, 64, 0, 0, 0, ctypes.byref(sch), ctypes.byref(splits)) == ERR_SHAPE
    assert lib.gba_split_plan(64, 64, 64, 6, 0, 0, ctypes.byref(sch), ctypes.byref(splits)) == ERR_ACT


def test_transpose_a_argument_errors_precede_device_use(lib):
    # A stored [K, M]: M is then a row pitch, so it must be a multiple of 8 (16-byte
    # rows) and at most 2^23, like N; the other checks are unchanged.
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    ex = lambda M=64, N=64, K=64, flags=4, A=P16, C=P16 * 64: lib.gemm_bias_act_ex(
        v(A), v(P16), None, v(C), M, N, K, 0, 0, flags, None, 0)
    assert ex(M=60) == ERR_ALIGN
    assert ex(M=60, flags=5) == ERR_ALIGN
    assert ex(M=60, flags=0) != ERR_ALIGN          # [M, K] layout: any M
    assert ex(M=(1 << 23) + 8, C=P16 * (1 << 20)) == ERR_SHAPE
    assert ex(K=12) == ERR_ALIGN
    assert ex(N=60) == ERR_ALIGN
    assert ex(A=P16 + 2) == ERR_ALIGN
    assert ex(flags=8) == ERR_SHAPE                # unknown flag bit
    assert ex(C=P16 + 64) == ERR_ALIAS             # C overlaps At
    assert ex(M=0) == OK
    size = ctypes.c_size_t(123)
    assert lib.gba_workspace_size(0, 64, 64, 0, 0, 4, ctypes.byref(size)) == OK and size.value == 0
    s = gba.Schedule()
    assert lib.gba_get_schedule_ex(64, 64, 64, 0, 0, 8, ctypes.byref(s)) == ERR_SHAPE
    assert lib.gba_get_schedule_ex(64, 64, 64, 6, 0, 4, ctypes.byref(s)) == ERR_ACT


def test_bias_act_argument_errors(lib):
    v = ctypes.c_void_p
    assert lib.bias_act(v(P16), None, v(P16), 4, 8, 6, 0) == ERR_ACT
    assert lib.bias_act(v(P16), None, v(P16), 4, 12, 0, 0) == ERR_ALIGN
    assert lib.bias_act(None, None, v(P16), 4, 8, 0, 0) == ERR_NULL
    assert lib.bias_act(v(P16), None, v(P16 + 16), 4, 8, 0, 0) == ERR_ALIAS   # partial overlap
    assert lib.bias_act(v(P16), v(P16 * 2 + 32), v(P16 * 2), 4, 8, 0, 0) == ERR_ALIAS
    assert lib.bias_act(v(P16), None, v(P16), 0, 8, 0, 0) == OK


def test_no_device_gives_device_error(lib):
    if _gpu_present():
        pytest.skip("a GPU is present; this checks the GPU-less path")
    assert call(lib) == ERR_DEVICE
    assert lib.bias_act(ctypes.c_void_p(P16), None, ctypes.c_void_p(P16), 4, 8, 0, 0) == ERR_DEVICE
    s = gba.Schedule()
    assert lib.gba_get_schedule(64, 64, 64, 0, 0, ctypes.byref(s)) == ERR_DEVICE


def test_binding_checks_without_gpu():
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        gba.gemm_bias_act(a, a.t().contiguous(), None, torch.zeros(4, 4, dtype=torch.float16))
    # transpose_a: a is [K, M], so a [4, 8] operand means M = 8, K = 4
    assert gba._gemm_shapes(a, torch.zeros(4, 16, dtype=torch.float16), None,
                            torch.zeros(8, 16, dtype=torch.float16), False, True)[1:] == (8, 16, 4)
    with pytest.raises(ValueError):
        gba._gemm_shapes(a, torch.zeros(8, 16, dtype=torch.float16), None,
                         torch.zeros(8, 16, dtype=torch.float16), False, True)
    with pytest.raises(TypeError):
        gba._dtype_code(torch.zeros(2, dtype=torch.float32))
