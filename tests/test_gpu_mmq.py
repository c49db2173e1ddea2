"""GPU parity for the prefill GEMM (MMQ) kernels against the fp64 oracle.

Sizes span one tile, ragged tiles in both dimensions, and the full prefill
shapes (4096 x 4096 at T = 512; 14336 x 4096 Q4_K and 4096 x 14336 Q6_K at
T = 1024 with 1% x20 activation outliers) in the launch configuration the
bench times.  The integer stage (int8 MFMA results before scaling) is
compared bit for bit, and against the matvec's integer stage.
"""
import numpy as np
import pytest

import oracle
import qmm_synth
from _gpu import assert_parity, dev, host, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu

FMTS = {
    "q4k": (qmm_synth.q4k_weights, oracle.q4k_dequant, qmm.mmq_q4k, qmm.QMM_Q4_K),
    "q5k": (qmm_synth.q5k_weights, oracle.q5k_dequant, qmm.mmq_q5k, qmm.QMM_Q5_K),
    "q6k": (qmm_synth.q6k_weights, oracle.q6k_dequant, qmm.mmq_q6k, qmm.QMM_Q6_K),
}


def _inputs(fmt, M, K, T, seed, outliers=0.0):
    g = qmm_synth.rng(seed)
    w = FMTS[fmt][0](g, M, K)
    x = qmm_synth.activations(g, T, K, outlier_frac=outliers)
    return w, oracle.quantize_q8_1(x)


def _check(fmt, w, xq, what):
    y = host(FMTS[fmt][2](dev(w), dev(xq)))
    W, X = FMTS[fmt][1](w), oracle.q8_1_dequant(xq)
    assert_parity(y, oracle.dense(W, X), oracle.abs_bound(W, X), what)
    return y


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", [(128, 256, 64), (130, 512, 65), (300, 768, 130), (1, 256, 1),
                                   (129, 1024, 1), (64, 512, 200), (517, 256, 33)])
def test_parity_small(fmt, M, K, T):
    w, xq = _inputs(fmt, M, K, T, seed=M * 3 + T)
    say(f"mmq_{fmt}", f"M={M} K={K} T={T}")
    _check(fmt, w, xq, f"mmq_{fmt} {M}x{K} T={T}")


def test_parity_prefill_4096x4096_t512():
    w, xq = _inputs("q4k", 4096, 4096, 512, seed=2)
    say("mmq_q4k", "M=4096 K=4096 T=512")
    _check("q4k", w, xq, "mmq_q4k 4096x4096 T=512")


@pytest.mark.parametrize("fmt,M,K", [("q4k", 14336, 4096), ("q6k", 4096, 14336)])
def test_parity_ffn_up_t1024(fmt, M, K):
    w, xq = _inputs(fmt, M, K, 1024, seed=3, outliers=0.01)
    say(f"mmq_{fmt}", f"M={M} K={K} T=1024 outliers")
    _check(fmt, w, xq, f"mmq_{fmt} {M}x{K} T=1024")


# Calls with few tiles split each tile's K range over several workgroups
# (partial tiles added in split order by the last one to finish): several
# splits with ragged step ranges, two column tiles per tile, one row, and
# the decode shape 4096 x 11008 at T = 8 and 32.
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", [(256, 4096, 8), (130, 2816, 33), (1, 11008, 1), (100, 11008, 3),
                                   (4096, 11008, 8), (4096, 11008, 32)])
def test_parity_split_k(fmt, M, K, T):
    w, xq = _inputs(fmt, M, K, T, seed=M + K + T)
    say(f"mmq_{fmt} split-K", f"M={M} K={K} T={T}")
    _check(fmt, w, xq, f"mmq_{fmt} {M}x{K} T={T}")


# Fused quantizer: fp32 activations quantized inside the call give the bytes
# of q8_1_quantize, so the output equals the Q8_1 path bit for bit (one
# tile, ragged tiles, split K, the 4096 x 4096 prefill shape), and the
# oracle on its own Q8_1 quantization.  Rows of zeros and 1 % outliers x20
# are included.
F32 = {"q4k": qmm.mmq_q4k_f32, "q5k": qmm.mmq_q5k_f32, "q6k": qmm.mmq_q6k_f32}


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", [(128, 256, 1), (130, 512, 65), (300, 768, 130), (256, 4096, 8),
                                   (4096, 4096, 512)])
def test_fused_quantizer_bit_identical(fmt, M, K, T):
    g = qmm_synth.rng(M + 7 * T)
    w = FMTS[fmt][0](g, M, K)
    x = qmm_synth.activations(g, T, K, outlier_frac=0.01)
    x[T // 2] = 0.0
    wd, xd = dev(w), dev(x)
    say(f"mmq_{fmt}_f32", f"M={M} K={K} T={T}")
    y1 = host(F32[fmt](wd, xd))
    y0 = host(FMTS[fmt][2](wd, qmm.q8_1_quantize(xd)))
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    if M * K * T <= 1 << 26:
        xq = oracle.quantize_q8_1(x)
        W, X = FMTS[fmt][1](w), oracle.q8_1_dequant(xq)
        assert_parity(y1, oracle.dense(W, X), oracle.abs_bound(W, X), f"mmq_{fmt}_f32 {M}x{K} T={T}")


def test_q5k_prefill_4096x4096_t512():
    w, xq = _inputs("q5k", 4096, 4096, 512, seed=5)
    say("mmq_q5k", "M=4096 K=4096 T=512")
    _check("q5k", w, xq, "mmq_q5k 4096x4096 T=512")


def test_split_k_deterministic():
    w, xq = _inputs("q6k", 4096, 11008, 16, seed=12)
    wd, xd = dev(w), dev(xq)
    say("mmq_q6k split-K determinism M=4096 K=11008 T=16")
    runs = [host(qmm.mmq_q6k(wd, xd)) for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(runs[0].view(np.uint32), r.view(np.uint32))


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", [(128, 256, 32), (150, 512, 70)])
def test_integer_stage_bit_exact(fmt, M, K, T):
    w, xq = _inputs(fmt, M, K, T, seed=M + 2 * T)
    say(f"debug_subdots path=1 {fmt}", f"M={M} K={K} T={T}")
    D, S = qmm.debug_subdots(FMTS[fmt][3], 1, dev(w), dev(xq))
    if fmt in ("q4k", "q5k"):
        Dr, Sr = (oracle.q4k_subdots if fmt == "q4k" else oracle.q5k_subdots)(w, xq)
        assert np.array_equal(host(S), Sr)
    else:
        Dr = oracle.q6k_subdots(w, xq)
    assert np.array_equal(host(D), Dr)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_matvec_and_gemm_integer_stages_agree(fmt):
    w, xq = _inputs(fmt, 96, 1024, 4, seed=9)
    say(f"debug_subdots path 0 vs 1 {fmt}", "M=96 K=1024 T=4")
    D0, S0 = qmm.debug_subdots(FMTS[fmt][3], 0, dev(w), dev(xq))
    D1, S1 = qmm.debug_subdots(FMTS[fmt][3], 1, dev(w), dev(xq))
    assert np.array_equal(host(D0), host(D1))
    if S0 is not None:
        assert np.array_equal(host(S0), host(S1))


def test_deterministic_and_repeated_calls():
    w, xq = _inputs("q4k", 1000, 2048, 300, seed=4)
    wd, xd = dev(w), dev(xq)
    say("mmq_q4k determinism M=1000 K=2048 T=300")
    runs = [host(qmm.mmq_q4k(wd, xd)) for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(runs[0].view(np.uint32), r.view(np.uint32))
    # a smaller call right after a larger one reuses the (self-resetting) workspace
    small = host(qmm.mmq_q4k(wd[:10].contiguous(), xd[:5].contiguous()))
    assert np.array_equal(small.view(np.uint32), runs[0][:5, :10].view(np.uint32))


def test_zero_scales_give_exact_zero():
    g = qmm_synth.rng(8)
    w = qmm_synth.q6k_weights(g, 130, 512)
    w[:, :, 192:208] = 0
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 40, 512))
    say("mmq_q6k zero scales")
    assert not host(qmm.mmq_q6k(dev(w), dev(xq))).any()
