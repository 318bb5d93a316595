"""The on-disk schedule cache, exercised without a GPU through gba_cache_store /
gba_cache_lookup (the same code the autotuner and every GEMM call use).

The pages' tuning cache ("TileLang: Write, Autotune, and Ship Fused
Tensor-Core Kernels from Python", Autotuning: how it works and how much it
costs) is reused by later runs, kept across CI, and switched off by an
environment variable. Here: missing, corrupt, stale (other build) and
unwritable caches, GBA_DISABLE_CACHE, a changed GBA_CACHE_DIR, and writers in
several processes.
"""
import json
import os
import subprocess
import sys

import pytest

import tiled_dense_gemm_bias_amd as gba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ARCH = "gfx950:sramecc+:xnack-"


@pytest.fixture
def cache_dir(tmp_path, monkeypatch):
    d = tmp_path / "gba-cache"
    monkeypatch.setenv("GBA_CACHE_DIR", str(d))
    monkeypatch.delenv("GBA_DISABLE_CACHE", raising=False)
    return d


def _scheds():
    s = gba.list_schedules()
    assert len(s) >= 2
    return s


def _keys(path):
    with open(path) as f:
        lines = f.read().splitlines()
    assert lines[0].startswith('{"format": "gba-schedule-cache", "version": 1')
    return [json.loads(l.rstrip(","))["key"] for l in lines[1:-1]]


def test_missing_cache_is_empty(cache_dir):
    assert gba.cache_lookup(ARCH, 256, 4096, 4096, 4096) is None
    assert not cache_dir.exists()   # a lookup creates nothing


def test_store_then_lookup_roundtrip(cache_dir):
    s0, s1 = _scheds()[:2]
    assert gba.cache_store(ARCH, 256, 4096, 4096, 4096, s0, 0.125) == 0
    assert gba.cache_store(ARCH, 256, 1024, 1024, 1024, s1, 0.011, act="none") == 0
    got = gba.cache_lookup(ARCH, 256, 4096, 4096, 4096)
    assert {k: got[k] for k in s0} == s0 and abs(got["ms"] - 0.125) < 1e-9
    got = gba.cache_lookup(ARCH, 256, 1024, 1024, 1024, act="none")
    assert {k: got[k] for k in s1} == s1
    # other act / dtype / layout / CU count / arch: different keys
    assert gba.cache_lookup(ARCH, 256, 1024, 1024, 1024, act="gelu") is None
    assert gba.cache_lookup(ARCH, 256, 4096, 4096, 4096, dtype="bf16") is None
    assert gba.cache_lookup(ARCH, 256, 4096, 4096, 4096, transpose_b=True) is None
    assert gba.cache_lookup(ARCH, 304, 4096, 4096, 4096) is None
    assert gba.cache_lookup("gfx942", 256, 4096, 4096, 4096) is None
    keys = _keys(cache_dir / "schedules.json")
    assert len(keys) == 2 and all(gba.build_id() in k for k in keys)


def test_corrupt_cache_is_ignored_and_replaced(cache_dir):
    cache_dir.mkdir()
    f = cache_dir / "schedules.json"
    s0 = _scheds()[0]
    good = dict(key="%s|256|%s|f16|gelu|nn|64|64|64" % (ARCH, gba.build_id()), ms=1.0, **s0)
    f.write_text('{"format": "gba-schedule-cache", "version": 1, "entries": [\n'
                 '{"key": "truncated|line", "bm": 25\n'
                 '\x00\xff garbage \n'
                 '{"key": "%s|256|%s|f16|gelu|nn|8|8|8", "bm": 1, "bn": 2, "bk": 3, "wm": 1, "wn": 1, '
                 '"stages": 2, "raster": 0, "group_m": 1, "kernel": 77, "loaders": 0, "spread": 0},\n'
                 % (ARCH, gba.build_id()) + json.dumps(good) + "\n")   # no closing bracket either
    got = gba.cache_lookup(ARCH, 256, 64, 64, 64)
    assert got is not None and {k: got[k] for k in s0} == s0   # the valid line survives
    assert gba.cache_lookup(ARCH, 256, 8, 8, 8) is None        # schedule not compiled in
    # A file of another format (or plain garbage) is ignored as a whole.
    f.write_text("not json at all\n" + json.dumps(good) + "\n")
    assert gba.cache_store(ARCH, 256, 32, 32, 32, s0, 2.0) == 0
    keys = _keys(f)
    assert keys == ["%s|256|%s|f16|gelu|nn|32|32|32" % (ARCH, gba.build_id())]


def test_stale_build_is_not_used_but_kept(cache_dir):
    cache_dir.mkdir()
    f = cache_dir / "schedules.json"
    s0 = _scheds()[0]
    stale_key = "%s|256|0123456789abcdef|f16|gelu|nn|4096|4096|4096" % ARCH
    f.write_text('{"format": "gba-schedule-cache", "version": 1, "entries": [\n'
                 + json.dumps(dict(key=stale_key, ms=0.1, **s0)) + "\n]}\n")
    assert gba.cache_lookup(ARCH, 256, 4096, 4096, 4096) is None
    assert gba.cache_store(ARCH, 256, 2048, 2048, 2048, s0, 0.05) == 0
    assert stale_key in _keys(f)   # another build's entry is preserved


def test_unwritable_cache_dir(tmp_path, monkeypatch):
    blocker = tmp_path / "a_file"
    blocker.write_text("x")
    monkeypatch.setenv("GBA_CACHE_DIR", str(blocker / "sub"))   # parent is a regular file
    monkeypatch.delenv("GBA_DISABLE_CACHE", raising=False)
    assert gba.cache_store(ARCH, 256, 64, 64, 64, _scheds()[0], 1.0) == 10   # GBA_ERR_CACHE
    assert gba.cache_lookup(ARCH, 256, 64, 64, 64) is None


def test_disable_cache(cache_dir, monkeypatch):
    s0 = _scheds()[0]
    assert gba.cache_store(ARCH, 256, 64, 64, 64, s0, 1.0) == 0
    monkeypatch.setenv("GBA_DISABLE_CACHE", "1")
    assert gba.cache_lookup(ARCH, 256, 64, 64, 64) is None          # not read
    assert gba.cache_store(ARCH, 256, 128, 128, 128, s0, 1.0) == 0  # not written
    monkeypatch.setenv("GBA_DISABLE_CACHE", "0")
    assert gba.cache_lookup(ARCH, 256, 64, 64, 64) is not None
    assert gba.cache_lookup(ARCH, 256, 128, 128, 128) is None


def test_changed_cache_dir_is_reread_and_not_merged(tmp_path, monkeypatch):
    monkeypatch.delenv("GBA_DISABLE_CACHE", raising=False)
    s0, s1 = _scheds()[:2]
    d1, d2 = tmp_path / "one", tmp_path / "two"
    monkeypatch.setenv("GBA_CACHE_DIR", str(d1))
    assert gba.cache_store(ARCH, 256, 64, 64, 64, s0, 1.0) == 0
    monkeypatch.setenv("GBA_CACHE_DIR", str(d2))
    assert gba.cache_lookup(ARCH, 256, 64, 64, 64) is None
    assert gba.cache_store(ARCH, 256, 128, 128, 128, s1, 1.0) == 0
    assert len(_keys(d2 / "schedules.json")) == 1    # d1's entry did not leak into d2
    monkeypatch.setenv("GBA_CACHE_DIR", str(d1))
    assert gba.cache_lookup(ARCH, 256, 64, 64, 64) is not None
    assert gba.cache_lookup(ARCH, 256, 128, 128, 128) is None


def _child(code, env):
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    return res.stdout.strip()


def test_other_processes_read_and_merge(cache_dir):
    s0, s1 = _scheds()[:2]
    env = dict(os.environ)
    # This process has loaded (and cached in memory) the file before the child writes.
    assert gba.cache_store(ARCH, 256, 64, 64, 64, s0, 1.0) == 0
    code = ("import tiled_dense_gemm_bias_amd as g, json; s = g.list_schedules()[1]; "
            "print(json.dumps(g.cache_lookup(%r, 256, 64, 64, 64))); "
            "print(g.cache_store(%r, 256, 96, 96, 96, s, 3.0))" % (ARCH, ARCH))
    out = _child(code, env).splitlines()
    assert json.loads(out[0])["bm"] == s0["bm"]   # the child reads what this process wrote
    assert out[1] == "0"
    # Now this process writes again: the child's entry must survive the merge.
    assert gba.cache_store(ARCH, 256, 128, 128, 128, s1, 2.0) == 0
    keys = _keys(cache_dir / "schedules.json")
    assert len(keys) == 3
    assert any("|96|96|96" in k for k in keys)


def test_concurrent_writers_lose_nothing(cache_dir):
    env = dict(os.environ)
    n, per = 4, 12
    code = ("import tiled_dense_gemm_bias_amd as g, sys; s = g.list_schedules()[0]; w = int(sys.argv[1]); "
            "[g.cache_store(%r, 256, 8 * (w * %d + i + 1), 64, 64, s, 1.0) for i in range(%d)]"
            % (ARCH, per, per))
    procs = [subprocess.Popen([sys.executable, "-c", code, str(w)], cwd=ROOT, env=env)
             for w in range(n)]
    assert all(p.wait(timeout=120) == 0 for p in procs)
    assert len(set(_keys(cache_dir / "schedules.json"))) == n * per


def test_cache_argument_errors(cache_dir):
    s0 = _scheds()[0]
    lib = gba.lib()
    S = gba.Schedule.from_dict(s0)
    import ctypes
    assert lib.gba_cache_lookup(None, 256, 64, 64, 64, 3, 0, 0, None, None) == 1
    assert lib.gba_cache_lookup(b'gfx950"x', 256, 64, 64, 64, 3, 0, 0, None, None) == 7
    assert lib.gba_cache_lookup(b"gfx950", 0, 64, 64, 64, 3, 0, 0, None, None) == 2
    assert lib.gba_cache_lookup(b"gfx950", 256, -1, 64, 64, 3, 0, 0, None, None) == 2
    assert lib.gba_cache_lookup(b"gfx950", 256, 64, 64, 64, 3, 0, 64, None, None) == 2
    assert lib.gba_cache_lookup(b"gfx950", 256, 64, 64, 64, 9, 0, 0, None, None) == 4
    assert lib.gba_cache_store(b"gfx950", 256, 64, 64, 64, 3, 0, 0, None, 1.0) == 1
    assert lib.gba_cache_store(b"gfx950", 256, 64, 64, 64, 3, 0, 0, ctypes.byref(S), -1.0) == 2
    assert lib.gba_cache_store(b"gfx950", 256, 64, 64, 64, 3, 0, 0, ctypes.byref(S),
                               float("nan")) == 2
    bad = dict(s0, bm=7)
    assert lib.gba_cache_store(b"gfx950", 256, 64, 64, 64, 3, 0, 0,
                               ctypes.byref(gba.Schedule.from_dict(bad)), 1.0) == 9
