"""Python binding of libgba, the gfx950 fused GEMM + bias + activation library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgba.so (see include/gba.h for the C ABI). PyTorch supplies device
memory and the current stream. There is no fallback: if libgba.so is missing
or the device is not a gfx950, the calls raise.

    import torch, tiled_dense_gemm_bias_amd as gba
    c = torch.empty(M, N, dtype=torch.float16, device="cuda")
    gba.gemm_bias_act(a, b, bias, c, act="gelu")     # c = gelu(a @ b + bias)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgba.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "gba.h")

ACTS = {"none": 0, "relu": 1, "sigmoid": 2, "gelu": 3, "softplus": 4, "gelu_tanh": 5}
STATUS = {
    0: "GBA_OK", 1: "GBA_ERR_NULL", 2: "GBA_ERR_SHAPE", 3: "GBA_ERR_DTYPE", 4: "GBA_ERR_ACT",
    5: "GBA_ERR_ALIGN", 6: "GBA_ERR_ALIAS", 7: "GBA_ERR_DEVICE", 8: "GBA_ERR_HIP",
    9: "GBA_ERR_SCHEDULE", 10: "GBA_ERR_CACHE", 11: "GBA_TUNE_INCOMPLETE", 12: "GBA_ERR_SCRATCH",
}
SCHED_FIELDS = ("bm", "bn", "bk", "wm", "wn", "stages", "raster", "group_m", "kernel", "loaders",
                "spread")


class GbaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(status, status),
                                                 _lib().gba_status_string(status).decode()))


class Schedule(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in SCHED_FIELDS]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f in SCHED_FIELDS}

    @classmethod
    def from_dict(cls, d: dict) -> "Schedule":
        s = cls()
        defaults = {"stages": 2, "raster": 1, "group_m": 4, "kernel": 3, "loaders": 4, "spread": 1}
        for f in SCHED_FIELDS:
            setattr(s, f, int(d.get(f, defaults.get(f, 0))))
        return s


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libgba.so is not built; run: python -m tiled_dense_gemm_bias_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        p, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "gemm_bias_act": [p, p, p, p, i64, i64, i64, ci, ci],
            "gemm": [p, p, p, i64, i64, i64, ci],
            "gemm_bias_act_nt": [p, p, p, p, i64, i64, i64, ci, ci],
            "gemm_nt": [p, p, p, i64, i64, i64, ci],
            "gemm_bias_act_fp8_nt": [p, p, p, p, i64, i64, i64, ctypes.c_float, ci, ci, ci],
            "gemm_bias_act_ex": [p, p, p, p, i64, i64, i64, ci, ci, ci, p, ctypes.c_size_t],
            "gemm_bias_act_fp8_ex": [p, p, p, p, i64, i64, i64, ctypes.c_float, ci, ci, ci, p,
                                     ctypes.c_size_t],
            "gba_workspace_size": [i64, i64, i64, ci, ci, ci, ctypes.POINTER(ctypes.c_size_t)],
            "gba_split_plan": [i64, i64, i64, ci, ci, ci, ctypes.POINTER(Schedule),
                               ctypes.POINTER(ci)],
            "bias_act": [p, p, p, i64, i64, ci, ci],
            "gba_set_stream": [p],
            "gba_set_schedule": [ctypes.POINTER(Schedule)],
            "gba_get_schedule": [i64, i64, i64, ci, ci, ctypes.POINTER(Schedule)],
            "gba_get_schedule_nt": [i64, i64, i64, ci, ci, ctypes.POINTER(Schedule)],
            "gba_get_schedule_ex": [i64, i64, i64, ci, ci, ci, ctypes.POINTER(Schedule)],
            "gba_num_schedules": [],
            "gba_list_schedule": [ci, ctypes.POINTER(Schedule)],
            "gba_autotune": [p, p, p, p, i64, i64, i64, ci, ci, ci, ctypes.POINTER(Schedule),
                             ctypes.POINTER(ctypes.c_double)],
            "gemm_bias_act_noalloc": [p, p, p, p, i64, i64, i64, ci, ci, ci],
            "gba_noalloc_scratch_bytes": [],
            "gba_autotune_num_trials": [],
            "gba_autotune_trial": [ci, ctypes.POINTER(Schedule), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ci)],
            "gba_build_id": [],
            "gba_cache_lookup": [ctypes.c_char_p, ci, i64, i64, i64, ci, ci, ci,
                                 ctypes.POINTER(Schedule), ctypes.POINTER(ctypes.c_double)],
            "gba_cache_store": [ctypes.c_char_p, ci, i64, i64, i64, ci, ci, ci,
                                ctypes.POINTER(Schedule), ctypes.c_double],
            "gba_epilogue_probe": [p, p, i64, ci],
            "gba_clock_probe": [p, ci, ci, p],
            "gba_status_string": [ci],
            "gba_last_hip_error": [],
            "gba_version": [],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ci
        lib.gba_status_string.restype = ctypes.c_char_p
        lib.gba_version.restype = ctypes.c_char_p
        lib.gba_build_id.restype = ctypes.c_char_p
        lib.gba_noalloc_scratch_bytes.restype = ctypes.c_size_t
        _LIB = lib
    return _LIB


def lib():
    """The raw ctypes handle of libgba.so (C ABI of include/gba.h)."""
    return _lib()


def header_functions() -> list:
    """Names of the functions include/gba.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def version() -> str:
    return _lib().gba_version().decode()


# ------------------------------------------------------------- helpers ----

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise TypeError("gba supports float16 and bfloat16 tensors, got %s" % t.dtype)


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("gba works on device tensors; got a %s tensor" % t.device)
        if not t.is_contiguous():
            raise ValueError("gba needs contiguous row-major tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s and %s" % (dev, t.device))
    return dev


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _act(act) -> int:
    if isinstance(act, str):
        return ACTS[act]
    return int(act)


def _call(fn_name: str, dev, *args):
    """Run entry point fn_name on dev's current stream. The library launches on
    the calling thread's current device, so it is switched only when the
    tensors live elsewhere (the switch and torch's stream object cost a few
    microseconds, as much as a small GEMM)."""
    torch = _torch()
    lib = _lib()
    C = torch._C
    if dev.index == C._cuda_getDevice():
        lib.gba_set_stream(C._cuda_getCurrentRawStream(dev.index))
        st = getattr(lib, fn_name)(*args)
    else:
        with torch.cuda.device(dev):
            lib.gba_set_stream(C._cuda_getCurrentRawStream(dev.index))
            st = getattr(lib, fn_name)(*args)
    if st != 0:
        raise GbaError(st, fn_name)


# ---------------------------------------------------------------- API ----

def _gemm_shapes(a, b, bias, c, transpose_b, transpose_a=False):
    """(dtype code, M, N, K) after the dtype and shape checks of the GEMM calls.
    a is [M,K], or [K,M] with transpose_a; b is [K,N], or [N,K] with transpose_b."""
    dt = _dtype_code(a)
    for t in (b, bias, c):
        if t is not None and _dtype_code(t) != dt:
            raise TypeError("all operands must share one dtype")
    M, K = tuple(a.shape)[::-1] if transpose_a else tuple(a.shape)
    N, K2 = tuple(b.shape) if transpose_b else tuple(b.shape)[::-1]
    if K2 != K or tuple(c.shape) != (M, N) or (bias is not None and tuple(bias.shape) != (N,)):
        raise ValueError("shape mismatch: a%s%s b%s%s bias%s c%s" % (
            tuple(a.shape), " (transpose_a)" if transpose_a else "",
            tuple(b.shape), " (transpose_b)" if transpose_b else "",
            None if bias is None else tuple(bias.shape), tuple(c.shape)))
    return dt, M, N, K


TRANSPOSE_B = 1
TRANSPOSE_A = 4


def _layout_flags(transpose_a, transpose_b) -> int:
    return (TRANSPOSE_A if transpose_a else 0) | (TRANSPOSE_B if transpose_b else 0)


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("the workspace is a contiguous device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def gemm_bias_act(a, b, bias, c, act="gelu", transpose_b=False, workspace=None,
                  transpose_a=False):
    """c[M,N] = act(a[M,K] @ b[K,N] + bias[N]); bias may be None. Returns c.

    transpose_b: b is stored [N,K] (a linear layer's weight) and c = act(a @ b.T + bias).
    transpose_a: a is stored [K,M] and c = act(a.T @ b + bias) (gemm_bias_act_ex
    with GBA_TRANSPOSE_A).
    workspace: optional device tensor of workspace_size(...) bytes that lets
    shapes with fewer tiles than CUs split K (gemm_bias_act_ex)."""
    dev = _check_dev(a, b, bias, c)
    dt, M, N, K = _gemm_shapes(a, b, bias, c, transpose_b, transpose_a)
    if workspace is not None or transpose_a:
        ws, nb = None, 0
        if workspace is not None:
            _check_dev(workspace)
            ws, nb = _ws_args(workspace)
        _call("gemm_bias_act_ex", dev, _ptr(a), _ptr(b), _ptr(bias), _ptr(c), M, N, K, _act(act),
              dt, _layout_flags(transpose_a, transpose_b), ws, nb)
        return c
    _call("gemm_bias_act_nt" if transpose_b else "gemm_bias_act", dev, _ptr(a), _ptr(b),
          _ptr(bias), _ptr(c), M, N, K, _act(act), dt)
    return c


INPUT_FP8 = 2


def gemm_bias_act_noalloc(a, b, bias, c, act="gelu", transpose_b=False, transpose_a=False):
    """gemm_bias_act with a split-K workspace from the library's static scratch
    (no allocation; for graph capture and serving loops). Returns c."""
    dev = _check_dev(a, b, bias, c)
    dt, M, N, K = _gemm_shapes(a, b, bias, c, transpose_b, transpose_a)
    _call("gemm_bias_act_noalloc", dev, _ptr(a), _ptr(b), _ptr(bias), _ptr(c), M, N, K, _act(act),
          dt, _layout_flags(transpose_a, transpose_b))
    return c


def workspace_size(M: int, N: int, K: int, act="gelu", dtype="f16", transpose_b=False,
                   fp8=False, transpose_a=False) -> int:
    """Bytes of split-K workspace gemm_bias_act (gemm_bias_act_fp8 with fp8) would
    use for this shape (0: no split)."""
    out = ctypes.c_size_t()
    flags = _layout_flags(transpose_a, transpose_b) | (INPUT_FP8 if fp8 else 0)
    st = _lib().gba_workspace_size(M, N, K, _act(act), 0 if dtype in ("f16", "float16") else 1,
                                   flags, ctypes.byref(out))
    if st != 0:
        raise GbaError(st, "gba_workspace_size")
    return int(out.value)


def split_plan(M: int, N: int, K: int, act="gelu", dtype="f16", transpose_b=False,
               transpose_a=False):
    """(schedule dict, splits) of a gemm_bias_act call with a workspace of
    workspace_size(...) bytes: K split `splits` ways on that schedule's tiles
    (splits 1: one kernel, the get_schedule choice)."""
    sched = Schedule()
    splits = ctypes.c_int()
    st = _lib().gba_split_plan(M, N, K, _act(act), 0 if dtype in ("f16", "float16") else 1,
                               _layout_flags(transpose_a, transpose_b), ctypes.byref(sched),
                               ctypes.byref(splits))
    if st != 0:
        raise GbaError(st, "gba_split_plan")
    return sched.as_dict(), int(splits.value)


def bind_gemm_bias_act(a, b, bias, c, act="gelu", transpose_b=False, workspace=None,
                       transpose_a=False):
    """Check and marshal the arguments once; return a no-argument callable that
    enqueues c = act(a @ b + bias) (a @ b.T with transpose_b, a.T @ b with
    transpose_a) on the stream current now (one C call per invocation). For tight
    loops such as benchmarks; the tensors must stay alive and unchanged in shape
    while the callable is used."""
    dev = _check_dev(a, b, bias, c)
    dt, M, N, K = _gemm_shapes(a, b, bias, c, transpose_b, transpose_a)
    torch = _torch()
    lib = _lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (_ptr(a), _ptr(b), _ptr(bias), _ptr(c), M, N, K, _act(act), dt)
    name = "gemm_bias_act_nt" if transpose_b else "gemm_bias_act"
    if workspace is not None or transpose_a:
        ws_args = (None, 0)
        if workspace is not None:
            _check_dev(workspace)
            ws_args = _ws_args(workspace)
        args = args + ((_layout_flags(transpose_a, transpose_b),) + ws_args)
        name = "gemm_bias_act_ex"
    fn = getattr(lib, name)
    set_stream = lib.gba_set_stream

    def launch():
        # The library's stream is per thread and shared by every entry point:
        # set it on each call, so that launches stay on the bound stream
        # whatever other calls, or another thread, did in between.
        set_stream(stream)
        st = fn(*args)
        if st != 0:
            raise GbaError(st, name)

    if torch.cuda.current_device() != dev.index:
        raise ValueError("bind on the tensors' device (torch.cuda.set_device first)")
    return launch


FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def _fp8_code(t, fmt) -> int:
    torch = _torch()
    if fmt is None:
        if t.dtype == torch.float8_e4m3fn:
            return 0
        if t.dtype == torch.float8_e5m2:
            return 1
        raise TypeError("8-bit operands are float8_e4m3fn / float8_e5m2 tensors, or uint8 "
                        "bit patterns with fmt given; got %s" % t.dtype)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2):
        raise TypeError("8-bit operand expected, got %s" % t.dtype)
    return FP8_FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def gemm_bias_act_fp8(a, w, bias, c, scale=1.0, act="gelu", fmt=None, workspace=None):
    """c[M,N] = act(scale * a[M,K] @ w[N,K].T + bias[N]) with 8-bit a and w.

    a, w: float8_e4m3fn / float8_e5m2 tensors (or uint8 bit patterns with fmt
    "e4m3" / "e5m2"), w stored [N,K]; bias (or None) and c: float16 or bfloat16.
    scale: the fp32 dequantization factor of the product. workspace: optional
    device tensor of workspace_size(..., fp8=True) bytes enabling split-K.
    Returns c."""
    dev = _check_dev(a, w, bias, c)
    fa, fw = _fp8_code(a, fmt), _fp8_code(w, fmt)
    if fa != fw:
        raise TypeError("a and w must share one 8-bit format")
    dt = _dtype_code(c)
    if bias is not None and _dtype_code(bias) != dt:
        raise TypeError("bias and c must share one dtype")
    M, K = a.shape
    N, K2 = w.shape
    if K2 != K or tuple(c.shape) != (M, N) or (bias is not None and tuple(bias.shape) != (N,)):
        raise ValueError("shape mismatch: a%s w%s c%s" % (tuple(a.shape), tuple(w.shape),
                                                          tuple(c.shape)))
    if workspace is not None:
        _check_dev(workspace)
        ws, nb = _ws_args(workspace)
        _call("gemm_bias_act_fp8_ex", dev, _ptr(a), _ptr(w), _ptr(bias), _ptr(c), M, N, K,
              float(scale), _act(act), fa, dt, ws, nb)
        return c
    _call("gemm_bias_act_fp8_nt", dev, _ptr(a), _ptr(w), _ptr(bias), _ptr(c), M, N, K,
          float(scale), _act(act), fa, dt)
    return c


def bind_gemm_bias_act_fp8(a, w, bias, c, scale=1.0, act="gelu", fmt=None, workspace=None):
    """bind_gemm_bias_act for the 8-bit-input call (same checks as gemm_bias_act_fp8)."""
    dev = _check_dev(a, w, bias, c)
    fa = _fp8_code(a, fmt)
    if _fp8_code(w, fmt) != fa:
        raise TypeError("a and w must share one 8-bit format")
    dt = _dtype_code(c)
    M, K = a.shape
    N, K2 = w.shape
    if K2 != K or tuple(c.shape) != (M, N) or (bias is not None and tuple(bias.shape) != (N,)):
        raise ValueError("shape mismatch")
    torch = _torch()
    if torch.cuda.current_device() != dev.index:
        raise ValueError("bind on the tensors' device (torch.cuda.set_device first)")
    lib = _lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    set_stream = lib.gba_set_stream
    args = (_ptr(a), _ptr(w), _ptr(bias), _ptr(c), M, N, K, float(scale), _act(act), fa, dt)
    fn = lib.gemm_bias_act_fp8_nt
    if workspace is not None:
        _check_dev(workspace)
        args = args + _ws_args(workspace)
        fn = lib.gemm_bias_act_fp8_ex

    def launch():
        set_stream(stream)   # per call, as in bind_gemm_bias_act
        st = fn(*args)
        if st != 0:
            raise GbaError(st, "gemm_bias_act_fp8_nt")

    return launch


def gemm(a, b, c, transpose_b=False, transpose_a=False):
    """c[M,N] = a[M,K] @ b[K,N] (a @ b.T for b [N,K] with transpose_b; a.T for a
    [K,M] with transpose_a), rounded to the operand dtype. Returns c."""
    if transpose_a:
        return gemm_bias_act(a, b, None, c, "none", transpose_b=transpose_b, transpose_a=True)
    dev = _check_dev(a, b, c)
    dt, M, N, K = _gemm_shapes(a, b, None, c, transpose_b)
    _call("gemm_nt" if transpose_b else "gemm", dev, _ptr(a), _ptr(b), _ptr(c), M, N, K, dt)
    return c


def bias_act(x, bias, y, act="gelu"):
    """y[M,N] = act(x[M,N] + bias[N]) elementwise; y may be x. Returns y."""
    dev = _check_dev(x, bias, y)
    dt = _dtype_code(x)
    M, N = x.shape
    if tuple(y.shape) != (M, N) or (bias is not None and tuple(bias.shape) != (N,)):
        raise ValueError("shape mismatch")
    if _dtype_code(y) != dt or (bias is not None and _dtype_code(bias) != dt):
        raise TypeError("all operands must share one dtype")
    _call("bias_act", dev, _ptr(x), _ptr(bias), _ptr(y), M, N, _act(act), dt)
    return y


def epilogue_probe(z, y, act="gelu"):
    """y = act(z) on float32 device tensors, by the GEMM epilogue's device code."""
    torch = _torch()
    dev = _check_dev(z, y)
    if z.dtype != torch.float32 or y.dtype != torch.float32 or z.numel() != y.numel():
        raise ValueError("epilogue_probe takes two float32 tensors of one size")
    _call("gba_epilogue_probe", dev, _ptr(z), _ptr(y), z.numel(), _act(act))
    return y


def clock_probe(out, n_wg: int = 1024, spin_us: int = 20) -> int:
    """Enqueue the shader-clock probe on the current stream: out (a device
    int64 tensor of 2 * n_wg) receives per workgroup (core clock cycles,
    wall-clock ticks); returns the wall clock's rate in kHz. Core MHz =
    cycles / ticks * kHz / 1000, once the stream has finished."""
    torch = _torch()
    dev = _check_dev(out)
    if out.dtype != torch.int64 or out.numel() != 2 * n_wg or not out.is_contiguous():
        raise ValueError("clock_probe takes a contiguous int64 tensor of 2 * n_wg")
    khz = ctypes.c_int(0)
    _call("gba_clock_probe", dev, _ptr(out), n_wg, spin_us, ctypes.byref(khz))
    return khz.value


def set_schedule(sched: Optional[dict]) -> None:
    """Force a schedule (dict of SCHED_FIELDS) for this thread; None clears it."""
    lib = _lib()
    if sched is None:
        st = lib.gba_set_schedule(None)
    else:
        s = Schedule.from_dict(sched)
        st = lib.gba_set_schedule(ctypes.byref(s))
    if st != 0:
        raise GbaError(st, "gba_set_schedule")


def get_schedule(M: int, N: int, K: int, act="gelu", dtype="f16", transpose_b=False,
                 transpose_a=False) -> dict:
    s = Schedule()
    st = _lib().gba_get_schedule_ex(M, N, K, _act(act), 0 if dtype in ("f16", "float16") else 1,
                                    _layout_flags(transpose_a, transpose_b), ctypes.byref(s))
    if st != 0:
        raise GbaError(st, "gba_get_schedule")
    return s.as_dict()


def list_schedules() -> list:
    lib = _lib()
    out = []
    for i in range(lib.gba_num_schedules()):
        s = Schedule()
        lib.gba_list_schedule(i, ctypes.byref(s))
        out.append(s.as_dict())
    return out


TUNE_ALL_GROUPS, TUNE_TRANSPOSE_B, TUNE_TRANSPOSE_A = 1, 2, 4


def autotune(a, b, bias, c, act="gelu", all_groups: bool = False, transpose_b=False,
             transpose_a=False):
    """Time every compiled-in schedule on these buffers; cache and return the best.

    Returns (schedule dict, median ms). c holds the winner's result.
    """
    dev = _check_dev(a, b, bias, c)
    dt, M, N, K = _gemm_shapes(a, b, bias, c, transpose_b, transpose_a)
    best = Schedule()
    ms = ctypes.c_double()
    torch = _torch()
    with torch.cuda.device(dev):
        lib = _lib()
        lib.gba_set_stream(ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        st = lib.gba_autotune(_ptr(a), _ptr(b), _ptr(bias), _ptr(c), M, N, K, _act(act), dt,
                              (TUNE_ALL_GROUPS if all_groups else 0)
                              | (TUNE_TRANSPOSE_B if transpose_b else 0)
                              | (TUNE_TRANSPOSE_A if transpose_a else 0),
                              ctypes.byref(best), ctypes.byref(ms))
    if st not in (0, 10, 11):
        raise GbaError(st, "gba_autotune")
    return best.as_dict(), ms.value


def autotune_status(a, b, bias, c, act="gelu", all_groups: bool = False, transpose_b=False,
                    transpose_a=False):
    """autotune, returning (status, schedule dict, median ms, trials): status 0
    (done, cached), 10 (cache not writable) or 11 (stopped at GBA_TUNE_BUDGET;
    progress kept in the tuning journal, call again to resume); trials as
    autotune_trials()."""
    dev = _check_dev(a, b, bias, c)
    dt, M, N, K = _gemm_shapes(a, b, bias, c, transpose_b, transpose_a)
    best = Schedule()
    ms = ctypes.c_double()
    torch = _torch()
    with torch.cuda.device(dev):
        lib = _lib()
        lib.gba_set_stream(ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        st = lib.gba_autotune(_ptr(a), _ptr(b), _ptr(bias), _ptr(c), M, N, K, _act(act), dt,
                              (TUNE_ALL_GROUPS if all_groups else 0)
                              | (TUNE_TRANSPOSE_B if transpose_b else 0)
                              | (TUNE_TRANSPOSE_A if transpose_a else 0),
                              ctypes.byref(best), ctypes.byref(ms))
    if st not in (0, 10, 11):
        raise GbaError(st, "gba_autotune")
    return st, best.as_dict(), ms.value, autotune_trials()


def autotune_trials() -> list:
    """Per-candidate results of this thread's last autotune: dicts of the
    schedule plus "ms" (median) and "resumed" (taken from the tuning journal)."""
    lib = _lib()
    out = []
    for i in range(lib.gba_autotune_num_trials()):
        s, ms, res = Schedule(), ctypes.c_double(), ctypes.c_int()
        st = lib.gba_autotune_trial(i, ctypes.byref(s), ctypes.byref(ms), ctypes.byref(res))
        if st != 0:
            raise GbaError(st, "gba_autotune_trial")
        out.append(dict(s.as_dict(), ms=ms.value, resumed=bool(res.value)))
    return out


def build_id() -> str:
    """Hash of the sources this library was compiled from (gba_build_id)."""
    return _lib().gba_build_id().decode()


def _cache_args(arch, cus, M, N, K, act, dtype, transpose_b, transpose_a):
    return (arch.encode() if isinstance(arch, str) else arch, int(cus), int(M), int(N), int(K),
            _act(act), {"f16": 0, "bf16": 1}[dtype] if isinstance(dtype, str) else int(dtype),
            _layout_flags(transpose_a, transpose_b))


def cache_lookup(arch, cus, M, N, K, act="gelu", dtype="f16", transpose_b=False,
                 transpose_a=False):
    """The cached schedule (dict with "ms") for these arguments, or None (no
    entry, or the cache is disabled). Needs no device."""
    s, ms = Schedule(), ctypes.c_double()
    st = _lib().gba_cache_lookup(*_cache_args(arch, cus, M, N, K, act, dtype, transpose_b,
                                              transpose_a), ctypes.byref(s), ctypes.byref(ms))
    if st == 9:
        return None
    if st != 0:
        raise GbaError(st, "gba_cache_lookup")
    return dict(s.as_dict(), ms=ms.value)


def cache_store(arch, cus, M, N, K, sched: dict, ms: float, act="gelu", dtype="f16",
                transpose_b=False, transpose_a=False) -> int:
    """Merge one entry into the schedule cache; returns the status (0, or 10 if
    the cache could not be written). Needs no device."""
    s = Schedule.from_dict(sched)
    st = _lib().gba_cache_store(*_cache_args(arch, cus, M, N, K, act, dtype, transpose_b,
                                             transpose_a), ctypes.byref(s), float(ms))
    if st not in (0, 10):
        raise GbaError(st, "gba_cache_store")
    return st
