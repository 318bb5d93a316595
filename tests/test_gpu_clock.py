"""The shader-clock probe that the benchmark uses to report the clock its
timed launches ran at: every workgroup reports, the wall-clock interval is at
least the requested spin, and the ratio gives a core clock within the range an
MI355X can run at. Argument errors come back as status codes."""
import ctypes

import numpy as np
import pytest

import tiled_dense_gemm_bias_amd as gba

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_clock_probe_reads_a_plausible_core_clock():
    import torch
    n_wg, spin_us = 1024, 10
    out = torch.zeros(2 * n_wg, dtype=torch.int64, device="cuda")
    khz = gba.clock_probe(out, n_wg, spin_us)
    torch.cuda.synchronize()
    v = out.cpu().numpy().reshape(-1, 2)
    assert 1000 <= khz <= 10_000_000, khz
    ticks = khz * spin_us // 1000
    assert (v[:, 1] >= ticks).all(), v[:, 1].min()          # every wave spun its interval
    assert (v[:, 1] < 100 * ticks).all(), v[:, 1].max()
    mhz = v[:, 0] / v[:, 1] * khz / 1000.0
    print("clock probe: median %.1f MHz (min %.1f, max %.1f), wall clock %d kHz"
          % (np.median(mhz), mhz.min(), mhz.max(), khz))
    assert 100.0 < np.median(mhz) < 3000.0


def test_clock_probe_argument_errors():
    import torch
    lib = gba.lib()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    khz = ctypes.c_int(0)
    p = ctypes.c_void_p(out.data_ptr())
    assert lib.gba_clock_probe(None, 1, 10, ctypes.byref(khz)) == 1
    assert lib.gba_clock_probe(p, 1, 10, None) == 1
    assert lib.gba_clock_probe(p, 0, 10, ctypes.byref(khz)) == 2
    assert lib.gba_clock_probe(p, 65537, 10, ctypes.byref(khz)) == 2
    assert lib.gba_clock_probe(p, 1, 0, ctypes.byref(khz)) == 2
    assert lib.gba_clock_probe(p, 1, 100001, ctypes.byref(khz)) == 2
    with pytest.raises(ValueError):
        gba.clock_probe(out, 4)
