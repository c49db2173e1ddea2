"""Smoke runs of the measurement hooks (ceiling probes): each launch completes,
leaves its sink untouched (the kernels only store for an improbable value),
and a timed launch yields a rate in a plausible range for the hardware."""
import pytest
import torch

from _gpu import DEV, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu


def _time(fn):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3


def _cus():
    return torch.cuda.get_device_properties(DEV).multi_processor_count


@pytest.mark.parametrize("wps", [2, 4])
def test_probe_mfma(wps):
    sink = torch.zeros((4,), dtype=torch.int32, device=DEV)
    iters = 4096
    say("qmm_probe_mfma", f"iters={iters} waves/SIMD={wps}")
    s = _time(lambda: qmm.probe_mfma(iters, wps, sink))
    tops = _cus() * wps * 4 * iters * 4 * 65536 / s / 1e12
    say("  int8 TOPS", round(tops, 1))
    assert 100 < tops < 6000
    assert not sink.any()


@pytest.mark.parametrize("mode", [1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_probe_mfma_epilogue(mode):
    sink = torch.zeros((4,), dtype=torch.int32, device=DEV)
    iters = 2048
    say("qmm_probe_mfma_epilogue", f"mode={mode} iters={iters}")
    s = _time(lambda: qmm.probe_mfma_epilogue(mode, iters, 2, sink))
    tops = _cus() * 2 * 4 * iters * 2 * 65536 / s / 1e12
    say("  int8 TOPS", round(tops, 1))
    assert 20 < tops < 6000
    assert not sink.any()


@pytest.mark.parametrize("u,grid", [(1, 0), (4, 0), (16, 0), (8, 1024)])
def test_probe_read_geom(u, grid):
    nbytes = 64 << 20
    buf = torch.zeros((nbytes,), dtype=torch.uint8, device=DEV)
    sink = torch.zeros((4,), dtype=torch.int32, device=DEV)
    say("qmm_probe_read_geom", f"bytes={nbytes} loads/thread={u} grid={grid}")
    s = _time(lambda: qmm.probe_read_geom(buf, nbytes, u, grid, sink))
    gbps = nbytes / s / 1e9
    say("  GB/s", round(gbps, 1))
    assert 100 < gbps < 20000
    assert not sink.any()
