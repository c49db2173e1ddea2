"""GPU parity for the decode matvec (MMVQ) kernels against the fp64 oracle.

fp32 outputs must satisfy |y - y_ref| <= 1e-4 * sum_k |w_ik| |x_tk| element
by element; the integer sub-block sums of the kernels' own integer stage must
match the oracle's exactly.  The full 4096 x 11008 decode shape is checked at
T = 1 and T = 4, in the launch configuration the bench uses.
"""
import numpy as np
import torch
import pytest

import oracle
import qmm_synth
from _gpu import assert_parity, dev, host, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu

FMTS = {
    "q4k": (qmm_synth.q4k_weights, oracle.q4k_dequant, qmm.mmvq_q4k, qmm.QMM_Q4_K),
    "q5k": (qmm_synth.q5k_weights, oracle.q5k_dequant, qmm.mmvq_q5k, qmm.QMM_Q5_K),
    "q6k": (qmm_synth.q6k_weights, oracle.q6k_dequant, qmm.mmvq_q6k, qmm.QMM_Q6_K),
}
CASES = [(1, 256, 1), (7, 512, 3), (37, 1280, 8), (64, 2304, 4), (5, 256, 2), (1024, 1024, 1),
         (129, 768, 5), (200, 1536, 6), (90, 2816, 7), (4096, 11008, 1), (4096, 11008, 4),
         # one token with rows longer than one LDS segment (two and three segments)
         (40, 14336, 1), (11, 12032, 1), (19, 30720, 1),
         # one token, Q6_K rows split between the LDS copy and registers: none, one and eight
         # super-blocks in registers, and a matrix not ending on a 16-byte boundary
         (8, 9728, 1), (24, 9984, 1), (16, 11776, 1), (8, 768, 1), (9, 11008, 1),
         # two to four tokens, Q4_K rows copied into LDS by 16-row workgroups: rows of one and
         # two segments, a single super-block, a partial last workgroup
         (33, 14336, 4), (17, 12288, 2), (19, 11776, 3), (3, 256, 4),
         # two to four tokens, Q6_K rows split between 16-row LDS copies and registers
         (16, 11008, 4), (24, 7168, 2), (8, 9728, 3), (40, 6144, 4),
         # five to eight tokens, Q4_K / Q5_K rows in two and three LDS segments
         (16, 11008, 8), (21, 14336, 6), (35, 11008, 5)]


def _inputs(fmt, M, K, T, seed):
    gen = FMTS[fmt][0]
    g = qmm_synth.rng(seed)
    w = gen(g, M, K)
    x = qmm_synth.activations(g, T, K)
    return w, x, oracle.quantize_q8_1(x)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", CASES)
def test_parity(fmt, M, K, T):
    w, x, xq = _inputs(fmt, M, K, T, seed=M + K + T)
    say(f"mmvq_{fmt}", f"M={M} K={K} T={T}")
    y = host(FMTS[fmt][2](dev(w), dev(xq)))
    W, X = FMTS[fmt][1](w), oracle.q8_1_dequant(xq)
    assert_parity(y, oracle.dense(W, X), oracle.abs_bound(W, X), f"mmvq_{fmt} {M}x{K} T={T}")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_end_to_end_from_fp32(fmt):
    # GPU quantizer feeding the GPU matvec, as in the decode step
    w, x, xq = _inputs(fmt, 300, 2048, 2, seed=5)
    say(f"q8_1_quantize + mmvq_{fmt}", "M=300 K=2048 T=2")
    y = host(FMTS[fmt][2](dev(w), qmm.q8_1_quantize(dev(x))))
    W, X = FMTS[fmt][1](w), oracle.q8_1_dequant(xq)
    assert_parity(y, oracle.dense(W, X), oracle.abs_bound(W, X), fmt)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,K,T", [(3, 256, 1), (9, 768, 4), (17, 512, 5), (21, 768, 6), (33, 1024, 8),
                                   (13, 12544, 1), (10, 11008, 1), (16, 11008, 1), (8, 11776, 1),
                                   (21, 14336, 2), (18, 11008, 3), (16, 11008, 4), (8, 7424, 2),
                                   (24, 11008, 6), (16, 7168, 8)])
def test_integer_stage_bit_exact(fmt, M, K, T):
    w, x, xq = _inputs(fmt, M, K, T, seed=7 * M + T)
    say(f"debug_subdots path=0 {fmt}", f"M={M} K={K} T={T}")
    D, S = qmm.debug_subdots(FMTS[fmt][3], 0, dev(w), dev(xq))
    if fmt in ("q4k", "q5k"):
        Dr, Sr = (oracle.q4k_subdots if fmt == "q4k" else oracle.q5k_subdots)(w, xq)
        assert np.array_equal(host(S), Sr)
    else:
        Dr = oracle.q6k_subdots(w, xq)
    assert np.array_equal(host(D), Dr)


def test_zero_scales_give_exact_zero():
    g = qmm_synth.rng(3)
    w = qmm_synth.q4k_weights(g, 16, 512)
    w[:, :, 4:16] = 0            # all sc = m = 0
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    say("mmvq_q4k zero scales")
    y = host(qmm.mmvq_q4k(dev(w), dev(xq)))
    assert not y.any()


def test_q5k_without_fifth_bits_equals_q4k():
    # Blocks whose fifth bits are zero: the Q5_K kernel's integer sums equal
    # the Q4_K kernel's on the same d, dmin, scales and values; the fp32
    # results (summed in another lane order: 11 vs 9 chunks per block) both
    # meet the Q4_K oracle.
    g = qmm_synth.rng(17)
    w5 = qmm_synth.q5k_weights(g, 300, 2304)
    w5[..., 16:48] = 0
    w4 = np.ascontiguousarray(np.concatenate([w5[..., 0:16], w5[..., 48:176]], axis=-1))
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 3, 2304))
    say("mmvq_q5k vs mmvq_q4k, zero fifth bits")
    D5, S5 = qmm.debug_subdots(qmm.QMM_Q5_K, 0, dev(w5), dev(xq))
    D4, S4 = qmm.debug_subdots(qmm.QMM_Q4_K, 0, dev(w4), dev(xq))
    assert np.array_equal(host(D5), host(D4)) and np.array_equal(host(S5), host(S4))
    W, X = oracle.q4k_dequant(w4), oracle.q8_1_dequant(xq)
    ref, bound = oracle.dense(W, X), oracle.abs_bound(W, X)
    assert_parity(host(qmm.mmvq_q5k(dev(w5), dev(xq))), ref, bound, "q5k zero fifth bits")
    assert_parity(host(qmm.mmvq_q4k(dev(w4), dev(xq))), ref, bound, "q4k")


def test_deterministic():
    w, x, xq = _inputs("q4k", 4096, 11008, 4, seed=11)
    wd, xd = dev(w), dev(xq)
    say("mmvq_q4k determinism 4096x11008 T=4")
    a = host(qmm.mmvq_q4k(wd, xd))
    b = host(qmm.mmvq_q4k(wd, xd))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# Paired one-token matvecs (one launch for two matrices on the same row): every
# format pair against the oracle and bit for bit against the single matvecs; ragged
# row counts (a partial last workgroup on either side), the decode shape, and
# shapes the Q6_K one-token kernel does not take (then two launches).
FMT_PAIRS = [(a, b) for a in ("q4k", "q5k", "q6k") for b in ("q4k", "q5k", "q6k")]
PAIR_CASES = ([(a, b, Ma, Mb, K) for a, b in FMT_PAIRS
               for Ma, Mb, K in [(72, 40, 2816), (9, 13, 256), (16, 24, 12288), (9, 8, 11008)]]
              # the decode shape for the pairs a decode step uses
              + [(a, b, 4096, 4096, 11008) for a, b in (("q6k", "q4k"), ("q4k", "q4k"))])


@pytest.mark.parametrize("fa,fb,Ma,Mb,K", PAIR_CASES)
def test_pair_matches_single_matvecs(fa, fb, Ma, Mb, K):
    g = qmm_synth.rng(Ma + 3 * Mb + K)
    wa, wb = FMTS[fa][0](g, Ma, K), FMTS[fb][0](g, Mb, K)
    x = qmm_synth.activations(g, 1, K)
    xq = oracle.quantize_q8_1(x)
    say("mmvq_pair", f"{fa} Ma={Ma} {fb} Mb={Mb} K={K}")
    dxq = dev(xq)
    ya, yb = qmm.mmvq_pair(FMTS[fa][3], dev(wa), FMTS[fb][3], dev(wb), dxq)
    ya, yb = host(ya), host(yb)
    assert np.array_equal(ya, host(FMTS[fa][2](dev(wa), dxq)))
    assert np.array_equal(yb, host(FMTS[fb][2](dev(wb), dxq)))
    X = oracle.q8_1_dequant(xq)
    rows = np.arange(Ma) if Ma <= 512 else np.random.default_rng(1).choice(Ma, 64, replace=False)
    Wa = FMTS[fa][1](wa[rows])
    assert_parity(ya[:, rows], oracle.dense(Wa, X), oracle.abs_bound(Wa, X), f"pair a {fa}")
    rows = np.arange(Mb) if Mb <= 512 else np.random.default_rng(2).choice(Mb, 64, replace=False)
    Wb = FMTS[fb][1](wb[rows])
    assert_parity(yb[:, rows], oracle.dense(Wb, X), oracle.abs_bound(Wb, X), f"pair b {fb}")


def test_pair_rejects_bad_arguments():
    g = qmm_synth.rng(3)
    w = dev(qmm_synth.q4k_weights(g, 8, 512))
    xq = qmm.q8_1_quantize(dev(qmm_synth.activations(g, 2, 512)))
    with pytest.raises(ValueError):
        qmm.mmvq_pair(qmm.QMM_Q4_K, w, qmm.QMM_Q4_K, w, xq)  # two rows
    y = torch.empty((1, 8), dtype=torch.float32, device=w.device)
    with pytest.raises(ValueError):
        qmm.mmvq_pair(qmm.QMM_Q4_K, w, qmm.QMM_Q4_K, w, xq[:1].contiguous(), out_a=y, out_b=y)
    with pytest.raises(ValueError):
        qmm.mmvq_pair(qmm.QMM_Q4_K, w, qmm.QMM_Q4_K, dev(qmm_synth.q4k_weights(g, 8, 768)), xq[:1].contiguous())
