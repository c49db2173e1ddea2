"""Pins for the oracle's Q6_K decoder and its sub-block sums (CPU only).

Anchors: the sentinel block of tests/golden/q6k_block.txt (``d`` at byte 208,
the generator pitfall of minfer ch. 06 "decode MMVQ: dp4a integer dot
products", section 3.3), bijectivity of the 1536 ql/qh bits, brute force over
bytes, and the factorisation into 16-weight sub-block integer sums.
"""
import numpy as np

import oracle
import qmm_synth
from _golden import hexbytes, load, pairs


def _golden():
    rec = load("q6k_block.txt")[0]
    blk = np.zeros((1, 1, 210), dtype=np.uint8)
    blk[0, 0, 0:128] = np.frombuffer(hexbytes(rec["ql"]), np.uint8)
    blk[0, 0, 128:192] = int(rec["qh_byte"], 16)
    blk[0, 0, 192:208] = np.frombuffer(hexbytes(rec["sc"]), np.uint8)
    blk[0, 0, 208:210] = np.frombuffer(hexbytes(rec["d"]), np.uint8)
    return rec, blk


def test_golden_elements():
    rec, blk = _golden()
    w = oracle.q6k_dequant(blk)[0]
    for e, v in pairs(rec["elements"]).items():
        assert w[e] == v, e
    d, sc, _ = oracle.q6k_fields(blk[0])
    assert d[0] == 1.0
    assert sc[0].tolist() == [1, -2, 3, -4, 5, -6, 7, -8, 9, -10, 11, -12, 13, -14, 15, -16]


def test_value_bits_used_once():
    # Each of the 1024 ql bits and 512 qh bits feeds exactly one weight's
    # 6-bit value, and each (weight, value bit) pair is fed exactly once.
    base = np.zeros((1, 210), dtype=np.uint8)
    _, _, q0 = oracle.q6k_fields(base)
    seen = set()
    for byte in range(192):
        for bit in range(8):
            b = base.copy()
            b[0, byte] ^= 1 << bit
            _, _, q = oracle.q6k_fields(b)
            delta = (q - q0)[0]
            nzi = np.flatnonzero(delta)
            assert nzi.size == 1
            v = int(delta[nzi[0]])
            assert v > 0 and v & (v - 1) == 0 and v < 64
            seen.add((int(nzi[0]), v.bit_length() - 1))
    assert len(seen) == 256 * 6


def test_scale_groups_of_16():
    blk = np.zeros((1, 1, 210), dtype=np.uint8)
    blk[0, 0, 208:210] = np.array([0x3C00], "<u2").view(np.uint8)
    blk[0, 0, 192:208] = np.arange(1, 17, dtype=np.int8).view(np.uint8)
    w = oracle.q6k_dequant(blk)[0]            # all q6 = 0 -> value -32 * sc
    assert np.array_equal(w, -32.0 * np.repeat(np.arange(1, 17), 16))


def _brute_force_q6k(blocks, xq):
    M, nb, _ = blocks.shape
    T = xq.shape[0]
    D = np.zeros((T, M, nb * 16), dtype=np.int64)
    for i in range(M):
        for b in range(nb):
            blk = blocks[i, b]
            for e in range(256):
                h, r = divmod(e, 128)
                g, l = divmod(r, 32)
                low = (int(blk[64 * h + 32 * (g % 2) + l]) >> (4 * (g // 2))) & 15
                hi = (int(blk[128 + 32 * h + l]) >> (2 * g)) & 3
                w = (low | hi << 4) - 32
                for t in range(T):
                    q = int(np.int8(xq[t, b * 8 + e // 32, 4 + e % 32]))
                    D[t, i, b * 16 + e // 16] += w * q
    return D


def test_subdots_brute_force():
    g = np.random.default_rng(8)
    blocks = qmm_synth.q6k_weights(g, 2, 512)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    assert np.array_equal(oracle.q6k_subdots(blocks, xq), _brute_force_q6k(blocks, xq))


def test_factored_identity_matches_dense():
    g = np.random.default_rng(12)
    blocks = qmm_synth.q6k_weights(g, 5, 1024)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 3, 1024, outlier_frac=0.05))
    W, X = oracle.q6k_dequant(blocks), oracle.q8_1_dequant(xq)
    y = oracle.dense(W, X)
    assert np.all(np.abs(y - oracle.q6k_factored(blocks, xq)) <= 1e-12 * oracle.abs_bound(W, X))


def test_midpoint_values_give_zero():
    # q6 = 32 everywhere (low4 = 0, hi2 = 2 in every pair) makes every weight 0.
    g = np.random.default_rng(4)
    blocks = qmm_synth.q6k_weights(g, 3, 512)
    blocks[:, :, 0:128] = 0
    blocks[:, :, 128:192] = 0xAA
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    assert not oracle.dense(oracle.q6k_dequant(blocks), oracle.q8_1_dequant(xq)).any()


def test_generator_puts_d_at_208():
    g = np.random.default_rng(0)
    blocks = qmm_synth.q6k_weights(g, 64, 2048)
    d, sc, _ = oracle.q6k_fields(blocks)
    assert np.all(np.isfinite(d)) and d.min() >= 0
    assert 0.006 < d.mean() < 0.010          # E|N(0, 0.01)| = 0.008
    assert sc.min() >= -64 and sc.max() <= 63
