"""Pins for the oracle's Q4_K decoder, dense product and integer sub-block sums (CPU only).

Anchors: the hand-packed block of tests/golden/q4k_block.txt, bijectivity of
the 96 packed scale bits, brute force over bytes on tiny inputs, and the
min-term factorisation of minfer ch. 06 "decode MMVQ: dp4a integer dot
products", section 2 (closed form).
"""
import numpy as np
import pytest

import oracle
import qmm_synth
from _golden import hexbytes, load, pairs


def _golden():
    rec = load("q4k_block.txt")[0]
    blk = np.frombuffer(hexbytes(rec["block"]), dtype=np.uint8).reshape(1, 1, 144)
    return rec, blk


def _q8_block(d16_bits, q):
    """One Q8_1 block assembled by hand from its fields (layout only)."""
    b = np.zeros(40, dtype=np.uint8)
    b[0:2] = np.array([d16_bits], dtype="<u2").view(np.uint8)
    b[4:36] = np.asarray(q, dtype=np.int8).view(np.uint8)
    b[36:40] = np.array([int(np.sum(q))], dtype="<i4").view(np.uint8)
    return b


def test_golden_fields_and_elements():
    rec, blk = _golden()
    d, dmin, sc, m, nib = oracle.q4k_fields(blk[0])
    assert d[0] == 0.5 and dmin[0] == 0.25
    assert sc[0].tolist() == [int(v) for v in rec["sc"].split()]
    assert m[0].tolist() == [int(v) for v in rec["m"].split()]
    w = oracle.q4k_dequant(blk)[0]
    for e, v in pairs(rec["elements"]).items():
        assert w[e] == v, e


def test_golden_all_ones_activation():
    rec, blk = _golden()
    xq = np.stack([_q8_block(0x3C00, np.ones(32, np.int64)) for _ in range(8)]).reshape(1, 8, 40)
    W = oracle.q4k_dequant(blk)
    X = oracle.q8_1_dequant(xq)
    assert oracle.dense(W, X)[0, 0] == float(rec["y_all_ones"])
    assert oracle.q4k_factored(blk, xq)[0, 0] == float(rec["y_all_ones"])


def test_scale_packing_uses_each_bit_once():
    # Flipping any one of the 96 packed bits changes exactly one of the 16
    # six-bit fields, by a power of two, and every (field, bit) is reached once.
    base = np.zeros((1, 144), dtype=np.uint8)
    _, _, sc0, m0, _ = oracle.q4k_fields(base)
    seen = set()
    for byte in range(12):
        for bit in range(8):
            b = base.copy()
            b[0, 4 + byte] ^= 1 << bit
            _, _, sc, m, _ = oracle.q4k_fields(b)
            delta = np.concatenate([(sc - sc0)[0], (m - m0)[0]])
            nzi = np.flatnonzero(delta)
            assert nzi.size == 1
            v = int(delta[nzi[0]])
            assert v > 0 and v & (v - 1) == 0 and v < 64
            seen.add((int(nzi[0]), v.bit_length() - 1))
    assert len(seen) == 96


def test_nibble_addressing_one_hot_value_bytes():
    # Setting one nibble of one value byte changes exactly the element that
    # the addressing rule names; all others stay at -dmin*m = 0.
    blk = np.zeros((1, 1, 144), dtype=np.uint8)
    blk[0, 0, 0:2] = np.array([0x3C00], "<u2").view(np.uint8)   # d = 1
    blk[0, 0, 4:8] = 1                                          # sc_0..3 = 1
    blk[0, 0, 12:16] = 1                                        # sc_4..7 = 1
    for n in (0, 5, 31, 32, 77, 127):
        for hi in (0, 1):
            b = blk.copy()
            b[0, 0, 16 + n] = (7 << 4) if hi else 7
            w = oracle.q4k_dequant(b)[0]
            pair, l = divmod(n, 32)
            e = 64 * pair + 32 * hi + l
            expect = np.zeros(256)
            expect[e] = 7.0
            assert np.array_equal(w, expect), (n, hi)


def _brute_force_q4k(blocks, xq):
    """Byte-level loops: every weight decoded from its own byte, every product summed."""
    M, nb, _ = blocks.shape
    T = xq.shape[0]
    D = np.zeros((T, M, nb * 8), dtype=np.int64)
    S = np.zeros((T, nb * 8), dtype=np.int64)
    for t in range(T):
        for s in range(nb * 8):
            S[t, s] = sum(int(np.int8(xq[t, s, 4 + l])) for l in range(32))
    for i in range(M):
        for b in range(nb):
            for j in range(8):
                for l in range(32):
                    byte = int(blocks[i, b, 16 + 32 * (j // 2) + l])
                    nib = (byte >> 4) if (j % 2) else (byte & 15)
                    for t in range(T):
                        q = int(np.int8(xq[t, b * 8 + j, 4 + l]))
                        D[t, i, b * 8 + j] += nib * q
    return D, S


def test_subdots_brute_force():
    g = np.random.default_rng(7)
    blocks = qmm_synth.q4k_weights(g, 3, 512)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    D, S = oracle.q4k_subdots(blocks, xq)
    Db, Sb = _brute_force_q4k(blocks, xq)
    assert np.array_equal(D, Db) and np.array_equal(S, Sb)
    _, _, _, qsum = oracle.q8_1_fields(xq)
    assert np.array_equal(S, qsum)          # S equals the stored sum


def test_factored_identity_matches_dense():
    g = np.random.default_rng(11)
    blocks = qmm_synth.q4k_weights(g, 5, 1024)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 3, 1024, outlier_frac=0.05))
    W, X = oracle.q4k_dequant(blocks), oracle.q8_1_dequant(xq)
    y = oracle.dense(W, X)
    yf = oracle.q4k_factored(blocks, xq)
    bound = oracle.abs_bound(W, X)
    assert np.all(np.abs(y - yf) <= 1e-12 * bound)


def test_one_hot_activation_returns_weight_column():
    g = np.random.default_rng(3)
    blocks = qmm_synth.q4k_weights(g, 4, 512)
    W = oracle.q4k_dequant(blocks)
    for e in (0, 31, 32, 300, 511):
        q = np.zeros((16, 32), np.int64)
        q[e // 32, e % 32] = 1
        xq = np.stack([_q8_block(0x3C00, q[s]) for s in range(16)]).reshape(1, 16, 40)
        y = oracle.dense(W, oracle.q8_1_dequant(xq))
        assert np.array_equal(y[0], W[:, e])
        assert np.array_equal(oracle.q4k_factored(blocks, xq)[0], W[:, e])


def test_zero_scales_give_zero():
    g = np.random.default_rng(5)
    blocks = qmm_synth.q4k_weights(g, 3, 512)
    blocks[:, :, 4:16] = 0
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    y = oracle.dense(oracle.q4k_dequant(blocks), oracle.q8_1_dequant(xq))
    assert not y.any()


def test_zero_nibbles_leave_only_min_term():
    g = np.random.default_rng(6)
    blocks = qmm_synth.q4k_weights(g, 3, 512)
    blocks[:, :, 16:] = 0
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    y = oracle.dense(oracle.q4k_dequant(blocks), oracle.q8_1_dequant(xq))
    d, dmin, sc, m, _ = oracle.q4k_fields(blocks)
    dx, _, _, qsum = oracle.q8_1_fields(xq)
    mins = (dmin[:, :, None] * m).reshape(3, -1)
    expect = -(dx * qsum) @ mins.T
    assert np.allclose(y, expect, rtol=1e-13, atol=0)


def test_generator_layout_sentinels():
    # The generator must put f16 d/dmin at 0/2: both decode to |N(0, 0.02)|
    # draws (non-negative, finite, spread near 0.02).
    g = np.random.default_rng(0)
    blocks = qmm_synth.q4k_weights(g, 64, 2048)
    d, dmin, _, _, _ = oracle.q4k_fields(blocks)
    for v in (d, dmin):
        assert np.all(np.isfinite(v)) and v.min() >= 0
        assert 0.012 < v.mean() < 0.020     # E|N(0, s)| = 0.798 s = 0.016


@pytest.mark.parametrize("bad", [(1, 1, 143), (2, 145)])
def test_rejects_wrong_block_size(bad):
    with pytest.raises(ValueError):
        oracle.q4k_fields(np.zeros(bad, np.uint8))
