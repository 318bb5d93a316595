"""Resources and instructions of the built gfx950 kernels, checked on the CPU.

The pages' tuning advice ("TileLang: Write, Autotune, and Ship Fused
Tensor-Core Kernels from Python", Debugging and introspection; Prioritized
checklist, item 4) is to look at the generated code for the matrix-core
instruction and the async copies, and at register usage and spills. Here the
gfx950 code objects are taken out of libgba.so (each translation unit's clang
offload bundle in the .hip_fatbin section) and read with llvm-readelf (the
AMDHSA kernel metadata) and llvm-objdump (the instructions):

  * every kernel: no scratch (no register spills to memory), LDS within the
    160 KiB of a CU, at most 512 vector registers (arch + accumulation);
  * every GEMM kernel uses the MFMA of its dtype;
  * the direct-to-LDS kernels load with buffer_load_dwordx4 ... lds, read A with
    ds_read_b128, gather the [K,N] B operand with ds_read_b64_tr_b16, and
    synchronise with s_barrier.
"""
import os
import re
import struct
import subprocess
from collections import defaultdict

import pytest

import tiled_dense_gemm_bias_amd as gba

LLVM = "/opt/rocm/llvm/bin"
pytestmark = pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "llvm-objdump")),
                                reason="ROCm LLVM tools not installed")


def _code_objects(tmp):
    so = gba.LIB_PATH
    out = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-S", "-W", so],
                         capture_output=True, text=True, check=True).stdout
    off = size = None
    for line in out.splitlines():
        parts = line.split()
        if ".hip_fatbin" in parts:
            i = parts.index(".hip_fatbin")
            off, size = int(parts[i + 3], 16), int(parts[i + 4], 16)
    assert off is not None, "no .hip_fatbin section"
    with open(so, "rb") as f:
        f.seek(off)
        data = f.read(size)
    paths = []
    for m in re.finditer(rb"__CLANG_OFFLOAD_BUNDLE__", data):
        s = m.start()
        (n,) = struct.unpack_from("<Q", data, s + 24)
        p = s + 32
        for _ in range(n):
            eo, es, tl = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tl].decode()
            p += tl
            if triple.endswith("gfx950"):
                path = os.path.join(tmp, "co%d.elf" % len(paths))
                with open(path, "wb") as f:
                    f.write(data[s + eo:s + eo + es])
                paths.append(path)
    assert paths, "no gfx950 code object"
    return paths


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("co"))
    meta, insts, seq = {}, defaultdict(set), defaultdict(list)
    for path in _code_objects(tmp):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", path],
                               capture_output=True, text=True, check=True).stdout
        cur = None
        for line in notes.splitlines():
            m = re.match(r"\s+\.(\w+):\s+(.*)$", line)
            if not m:
                continue
            key, val = m.groups()
            if key == "name" and not val.endswith(".kd"):
                cur = meta.setdefault(val.strip(), {})
            elif cur is not None and key in ("private_segment_fixed_size", "group_segment_fixed_size",
                                             "vgpr_count", "agpr_count", "sgpr_count",
                                             "vgpr_spill_count", "sgpr_spill_count"):
                cur[key] = int(val)
        dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950",
                              "--no-show-raw-insn", path],
                             capture_output=True, text=True, check=True).stdout
        sym = None
        for line in dis.splitlines():
            m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
            if m:
                sym = m.group(1)
                continue
            if sym is None:
                continue
            t = line.strip().split()
            if t and re.match(r"^[a-z_][a-z0-9_]*$", t[0]):
                insts[sym].add(t[0] + (" lds" if t[0].startswith("buffer_load") and "lds" in t else ""))
                seq[sym].append(t[0])
    assert meta
    return meta, insts, seq


def _kind(name):
    for k in ("gemm_v5_kernel", "gemm_v3_kernel", "gemm_f8_kernel", "gemm_bias_act_kernel",
              "bias_act_kernel", "splitk_reduce_kernel", "epilogue_probe_kernel",
              "clock_probe_kernel"):
        if k in name:
            return k
    return None


def _targs(name):
    """Template arguments of a mangled kernel name, in order (ints and bools)."""
    body = name[name.index("ILi"):] if "ILi" in name else name
    return [int(v) for v in re.findall(r"L[ib](\d+)E", body)]


def test_every_kernel_is_known(kernels):
    meta, _, _ = kernels
    unknown = [n for n in meta if _kind(n) is None]
    assert not unknown, unknown
    kinds = {_kind(n) for n in meta}
    assert {"gemm_v5_kernel", "gemm_v3_kernel", "gemm_f8_kernel", "gemm_bias_act_kernel",
            "bias_act_kernel", "splitk_reduce_kernel"} <= kinds


def test_no_scratch_and_resources_fit(kernels):
    meta, _, _ = kernels
    bad = []
    for name, m in meta.items():
        if m.get("private_segment_fixed_size", 0) != 0 or m.get("vgpr_spill_count", 0) != 0:
            bad.append((name, m))
        assert m.get("group_segment_fixed_size", 0) <= 160 * 1024, (name, m)
        assert m.get("vgpr_count", 0) <= 512, (name, m)
    assert not bad, "kernels with scratch / spilled VGPRs: %s" % bad


def test_gemm_kernels_use_the_matrix_cores(kernels):
    meta, insts, _ = kernels
    for name in meta:
        kind = _kind(name)
        ins = insts[name]
        if kind == "gemm_f8_kernel":
            assert "v_mfma_f32_16x16x128_f8f6f4" in ins, name
        elif kind in ("gemm_v5_kernel", "gemm_v3_kernel"):
            dt = _targs(name)[4] if kind == "gemm_v5_kernel" else _targs(name)[9]
            want = "v_mfma_f32_16x16x32_" + ("f16" if dt == 0 else "bf16")
            assert want in ins, (name, sorted(i for i in ins if "mfma" in i))
            assert not any(i.startswith("v_mfma") and i != want for i in ins), name
        elif kind == "gemm_bias_act_kernel":
            dt = _targs(name)[5]
            assert "v_mfma_f32_32x32x16_" + ("f16" if dt == 0 else "bf16") in ins, name


def test_direct_to_lds_kernels_instruction_mix(kernels):
    meta, insts, _ = kernels
    seen = 0
    for name in meta:
        kind = _kind(name)
        if kind not in ("gemm_v5_kernel", "gemm_v3_kernel"):
            continue
        a = _targs(name)
        tb, ta = (a[6], a[7]) if kind == "gemm_v5_kernel" else (a[11], a[13])
        ins = insts[name]
        assert "buffer_load_dwordx4 lds" in ins, name
        assert "s_barrier" in ins, name
        # [M,K] A and [N,K] W are K-contiguous: 16-byte reads; [K,N] B and [K,M]
        # At are gathered with the transposing read
        if not ta or tb:
            assert "ds_read_b128" in ins, name
        if not tb or ta:
            assert "ds_read_b64_tr_b16" in ins, name
        assert not any(i.startswith("scratch_") for i in ins), name
        seen += 1
    assert seen >= 100


def test_persistent_main_loop_keeps_accumulators_in_place(kernels):
    """In the persistent kernel's first 128 MFMAs (one 64-deep slice of the
    main loop: 2 steps of 8x8 16x16x32 MFMAs per wave) no accumulator is copied
    or rewritten (v_accvgpr_mov / v_accvgpr_write) and nothing touches scratch:
    a register allocation that shuffles accumulators there costs the matrix core
    every slice even when the kernel has no scratch at all."""
    meta, _, seq = kernels
    seen = 0
    for name in meta:
        if _kind(name) != "gemm_v5_kernel":
            continue
        ops = seq[name]
        mf = [i for i, op in enumerate(ops) if op.startswith("v_mfma")]
        assert len(mf) >= 128, name
        loop = ops[mf[0]:mf[127]]
        bad = [op for op in loop if op.startswith(("v_accvgpr_mov", "v_accvgpr_write", "scratch_"))]
        assert not bad, (name, sorted(set(bad)))
        seen += 1
    assert seen >= 40


def test_tile_kernel_main_loops_keep_accumulators_in_place(kernels):
    """In kernel 3's first slice (2 steps of (BM/WM/16) x (BN/WN/16) 16x16x32
    MFMAs per wave, the main loop) no accumulator is read, copied or rewritten
    (v_accvgpr_*): split-K first passes and fused instances alike. A register
    allocation that moves accumulators between register files there costs
    every slice (the split-K pass once did 96 such moves per slice)."""
    meta, _, seq = kernels
    seen = 0
    for name in meta:
        if _kind(name) != "gemm_v3_kernel":
            continue
        a = _targs(name)
        bm, bn, wm, wn, ms = a[0], a[1], a[3], a[4], a[8]
        if ms != 16:
            continue
        per_slice = 2 * (bm // wm // 16) * (bn // wn // 16)
        ops = seq[name]
        mf = [i for i, op in enumerate(ops) if op.startswith("v_mfma")]
        assert len(mf) >= per_slice, name
        loop = ops[mf[0]:mf[per_slice - 1]]
        bad = [op for op in loop if op.startswith(("v_accvgpr", "scratch_"))]
        assert not bad, (name, sorted(set(bad)))
        seen += 1
    assert seen >= 40


def test_fp8_main_loops_keep_accumulators_in_place(kernels):
    """The 8-bit persistent kernel's two slice bodies in the code (a tile's
    first slice, whose MFMAs start from zero, and the steady slice: 64
    16x16x128 MFMAs per wave each) neither copy nor rewrite an accumulator
    (v_accvgpr_mov / v_accvgpr_write) nor touch scratch, for every format,
    output dtype, activation and split-K first pass."""
    meta, _, seq = kernels
    seen = 0
    for name in meta:
        if _kind(name) != "gemm_f8_kernel":
            continue
        ops = seq[name]
        mf = [i for i, op in enumerate(ops) if op.startswith("v_mfma")]
        assert len(mf) >= 128, name
        for lo, hi in ((0, 63), (64, 127)):
            body = ops[mf[lo]:mf[hi]]
            assert sum(op.startswith("v_mfma") for op in body) == hi - lo, name
            bad = [op for op in body if op.startswith(("v_accvgpr_mov", "v_accvgpr_write", "scratch_"))]
            assert not bad, (name, lo, sorted(set(bad)))
        seen += 1
    assert seen >= 26
