"""GPU parity: the Q8_1 quantizer must reproduce the oracle's bytes exactly."""
import numpy as np
import pytest

import oracle
import qmm_synth
from _golden import hexbytes, load, pairs
from _gpu import dev, host, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu


def _special_blocks(x):
    """Overwrite a few blocks of row 0 with edge cases (zero, f16-subnormal d, exact ties, tiny scales)."""
    if x.shape[1] >= 128:
        x[0, 0:32] = 0.0
        g = np.random.default_rng(5)
        x[0, 32:64] = (g.standard_normal(32) * 1e-5).astype(np.float32)
        k = np.arange(-16, 16, dtype=np.float32) + np.float32(0.5)
        k[0] = 127.0
        x[0, 64:96] = k * np.float32(2.0**-3)
        x[0, 96:128] = -x[0, 64:96]
    if x.shape[1] >= 192:
        # fp32-subnormal scale (stored as zeros) and the smallest normal scale
        x[0, 128:160] = np.float32(0.0)
        x[0, 128] = np.float32(127 * 2.0**-127)
        x[0, 129] = np.float32(-3.0e-37)
        x[0, 160:192] = np.float32(0.0)
        x[0, 160] = np.float32(127 * 2.0**-126)
        x[0, 161] = np.float32(-63.5 * 2.0**-126)
    return x


def test_golden_blocks():
    recs = load("q8_1_blocks.txt")
    x = np.zeros((1, 32 * len(recs)), np.float32)
    for i, r in enumerate(recs):
        for k, v in pairs(r.get("x", "")).items():
            x[0, 32 * i + k] = np.float32(v)
    say("q8_1_quantize golden", len(recs), "blocks")
    got = host(qmm.q8_1_quantize(dev(x))).reshape(len(recs), 40)
    for i, r in enumerate(recs):
        assert got[i].tobytes() == hexbytes(r["bytes"]), r["name"]


@pytest.mark.parametrize("T,K,outliers", [
    (1, 32, 0.0), (1, 1024, 0.0), (1, 11008, 0.0), (4, 11008, 0.0), (7, 2080, 0.05),
    (512, 4096, 0.0), (1024, 4096, 0.01), (1024, 14336, 0.01), (4096, 768, 0.0),
])
def test_bit_exact(T, K, outliers):
    g = qmm_synth.rng(1000 + T + K)
    x = _special_blocks(qmm_synth.activations(g, T, K, outlier_frac=outliers))
    say("q8_1_quantize", f"T={T} K={K} outliers={outliers}")
    got = host(qmm.q8_1_quantize(dev(x)))
    ref = oracle.quantize_q8_1(x)
    if not np.array_equal(got, ref):
        bad = np.argwhere((got != ref).any(axis=-1))
        t, b = bad[0]
        raise AssertionError(f"{len(bad)} blocks differ; first (t={t}, block={b}): "
                             f"gpu={got[t, b].tolist()} ref={ref[t, b].tolist()}")


def test_deterministic_and_empty():
    g = qmm_synth.rng(77)
    x = dev(qmm_synth.activations(g, 33, 4096, outlier_frac=0.01))
    a = host(qmm.q8_1_quantize(x))
    b = host(qmm.q8_1_quantize(x))
    assert np.array_equal(a, b)
    e = qmm.q8_1_quantize(dev(np.zeros((0, 64), np.float32)))
    assert tuple(e.shape) == (0, 2, 40)
