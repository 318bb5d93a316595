"""Several host threads calling the library at once, each on its own stream.

The C ABI keeps per-thread state beside state that all threads share:
- per thread: the stream of gba_set_stream, the schedule of gba_set_schedule;
- shared: the device properties, the schedule cache, the static scratch of the
  allocation-free entry point.

Eight threads each get their own stream, output buffers and workload. The
workloads cover heuristic schedules, a forced schedule in two threads, split-K
with a caller's workspace, split-K through the allocation-free entry point
(one thread only: calls on that array must not overlap), and the [N,K] and
[K,M] layouts. Each thread makes 24 calls, rotating over three output buffers,
and other threads' calls run in between. Every output must equal, bit for
bit, the same call made alone beforehand on the default stream.
"""
import threading

import numpy as np
import pytest

import synth
import tiled_dense_gemm_bias_amd as gba
from tests.gpu_util import empty, say, to_bits, to_dev

pytestmark = pytest.mark.gpu

# (M, N, K, act, dtype, transpose_a, transpose_b, mode); mode: "heur", "forced",
# "ws" (caller's workspace) or "noalloc"
CASES = [
    (512, 512, 512, "gelu", "f16", False, False, "heur"),
    (300, 264, 1000, "relu", "bf16", False, True, "heur"),
    (256, 256, 4096, "none", "f16", False, False, "ws"),
    (520, 776, 600, "sigmoid", "bf16", True, False, "heur"),
    (1024, 1024, 1024, "gelu_tanh", "f16", False, False, "forced"),
    (129, 136, 4104, "softplus", "bf16", False, False, "noalloc"),
    (768, 768, 512, "gelu", "f16", False, False, "forced"),
    (2048, 2048, 256, "none", "bf16", False, False, "heur"),
]
CALLS = 24


@pytest.fixture(scope="module")
def setup():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    scheds = gba.list_schedules()
    data = []
    for i, (M, N, K, act, dt, ta, tb, mode) in enumerate(CASES):
        A = synth.random_bits((K, M) if ta else (M, K), dt, 9100 + i)
        B = synth.random_bits((N, K) if tb else (K, N), dt, 9200 + i, scale=1.0 / np.sqrt(K))
        bias = synth.random_bits((N,), dt, 9300 + i)
        sched = scheds[(3 * i) % len(scheds)] if mode == "forced" else None
        data.append(dict(a=to_dev(A, dt), b=to_dev(B, dt), bias=to_dev(bias, dt), sched=sched))
    torch.cuda.synchronize()
    yield torch, data
    gba.set_schedule(None)


def _run(torch, i, d, out, ws):
    M, N, K, act, dt, ta, tb, mode = CASES[i]
    if mode == "noalloc":
        gba.gemm_bias_act_noalloc(d["a"], d["b"], d["bias"], out, act, transpose_b=tb, transpose_a=ta)
    else:
        gba.gemm_bias_act(d["a"], d["b"], d["bias"], out, act, transpose_b=tb, transpose_a=ta,
                          workspace=ws)


def _workspace(torch, i):
    M, N, K, act, dt, ta, tb, mode = CASES[i]
    if mode != "ws":
        return None
    nb = gba.workspace_size(M, N, K, act, dt, transpose_b=tb, transpose_a=ta)
    assert nb > 0, "this case is meant to split K"
    return torch.empty(nb, dtype=torch.uint8, device="cuda")


def test_threads_on_their_own_streams_match_single_calls(setup):
    torch, data = setup
    # references: each call alone, default stream
    refs = []
    for i, d in enumerate(data):
        M, N = CASES[i][0], CASES[i][1]
        out = empty((M, N), CASES[i][4], fill_bits=0x7E00)
        say("thread reference", CASES[i], d["sched"])
        gba.set_schedule(d["sched"])
        try:
            _run(torch, i, d, out, _workspace(torch, i))
        finally:
            gba.set_schedule(None)
        torch.cuda.synchronize()
        refs.append(to_bits(out))
        assert not (refs[-1] == 0x7E00).any()

    results, errors = [None] * len(CASES), []
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            d = data[i]
            M, N = CASES[i][0], CASES[i][1]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [empty((M, N), CASES[i][4], fill_bits=0x7E00) for _ in range(3)]
                ws = _workspace(torch, i)
                gba.set_schedule(d["sched"])   # this thread's only
                start.wait()
                for k in range(CALLS):
                    _run(torch, i, d, outs[k % 3], ws)
                gba.set_schedule(None)
            s.synchronize()
            results[i] = [to_bits(o) for o in outs]
        except Exception as e:   # reported in the main thread
            errors.append((i, repr(e)))
            start.abort()

    say("threads", len(CASES), "x", CALLS, "calls")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, outs in enumerate(results):
        for k, got in enumerate(outs):
            assert np.array_equal(got, refs[i]), (CASES[i], k)
