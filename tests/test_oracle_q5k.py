"""Pins for the oracle's Q5_K decoder, dense product and integer sub-block sums (CPU only).

The pages name Q5_K as a third k-quant with matvec kernels of its own
(minfer ch. 06 "decode MMVQ: dp4a integer dot products", sections 1 and 6)
but do not give its layout; the oracle reads it as GGUF's Q5_K.  Anchors: the
hand-packed block of tests/golden/q5k_block.txt, bijectivity of the 1280
value bits, the reduction to Q4_K when the fifth bits are zero (and a shift
of 16*d*sc when they are all set), brute force over bytes on tiny inputs,
and the min-term factorisation of section 2 (closed form).
"""
import numpy as np
import pytest

import oracle
import qmm_synth
from _golden import hexbytes, load, pairs


def _golden():
    rec = load("q5k_block.txt")[0]
    blk = np.frombuffer(hexbytes(rec["block"]), dtype=np.uint8).reshape(1, 1, 176)
    return rec, blk


def _q8_block(d16_bits, q):
    b = np.zeros(40, dtype=np.uint8)
    b[0:2] = np.array([d16_bits], dtype="<u2").view(np.uint8)
    b[4:36] = np.asarray(q, dtype=np.int8).view(np.uint8)
    b[36:40] = np.array([int(np.sum(q))], dtype="<i4").view(np.uint8)
    return b


def test_golden_fields_and_elements():
    rec, blk = _golden()
    d, dmin, sc, m, q5 = oracle.q5k_fields(blk[0])
    assert d[0] == 0.5 and dmin[0] == 0.25
    assert sc[0].tolist() == [int(v) for v in rec["sc"].split()]
    assert m[0].tolist() == [int(v) for v in rec["m"].split()]
    assert q5.min() >= 0 and q5.max() <= 31
    w = oracle.q5k_dequant(blk)[0]
    for e, v in pairs(rec["elements"]).items():
        assert w[e] == v, e


def test_golden_all_ones_activation():
    rec, blk = _golden()
    xq = np.stack([_q8_block(0x3C00, np.ones(32, np.int64)) for _ in range(8)]).reshape(1, 8, 40)
    W = oracle.q5k_dequant(blk)
    X = oracle.q8_1_dequant(xq)
    assert oracle.dense(W, X)[0, 0] == float(rec["y_all_ones"])
    assert oracle.q5k_factored(blk, xq)[0, 0] == float(rec["y_all_ones"])


def test_value_bits_used_once():
    # Each of the 160 value bytes' 1280 bits moves exactly one element's q5
    # by a power of two below 32, and every (element, bit) is reached once:
    # 4 bits from qs and 1 from qh per element.
    base = np.zeros((1, 176), dtype=np.uint8)
    *_, q0 = oracle.q5k_fields(base)
    seen = set()
    for byte in range(16, 176):
        for bit in range(8):
            b = base.copy()
            b[0, byte] ^= 1 << bit
            *_, q = oracle.q5k_fields(b)
            delta = (q - q0)[0]
            nzi = np.flatnonzero(delta)
            assert nzi.size == 1, (byte, bit)
            v = int(delta[nzi[0]])
            assert v > 0 and v & (v - 1) == 0 and v < 32
            seen.add((int(nzi[0]), v.bit_length() - 1))
    assert len(seen) == 256 * 5


def test_fifth_bit_addressing():
    # Bit j of qh[l] is the fifth bit of element 32*j + l, nothing else.
    for l in (0, 7, 31):
        for j in range(8):
            b = np.zeros((1, 176), dtype=np.uint8)
            b[0, 16 + l] = 1 << j
            *_, q = oracle.q5k_fields(b)
            expect = np.zeros(256, np.int64)
            expect[32 * j + l] = 16
            assert np.array_equal(q[0], expect), (l, j)


def _as_q4k(blocks5):
    """The Q4_K block with the same d, dmin, scale bytes and 4-bit values (layout only)."""
    b4 = np.empty(blocks5.shape[:-1] + (144,), np.uint8)
    b4[..., 0:16] = blocks5[..., 0:16]
    b4[..., 16:144] = blocks5[..., 48:176]
    return b4


def test_reduces_to_q4k_without_fifth_bits():
    g = np.random.default_rng(13)
    b5 = qmm_synth.q5k_weights(g, 3, 512)
    b5[..., 16:48] = 0
    assert np.array_equal(oracle.q5k_dequant(b5), oracle.q4k_dequant(_as_q4k(b5)))
    # all fifth bits set: every weight moves by 16 * d * sc_j
    b5[..., 16:48] = 255
    d, _, sc, _, _ = oracle.q5k_fields(b5)
    shift = np.repeat((16.0 * d[..., None] * sc).reshape(3, -1), 32, axis=-1)
    assert np.array_equal(oracle.q5k_dequant(b5), oracle.q4k_dequant(_as_q4k(b5)) + shift)


def _brute_force_q5k(blocks, xq):
    M, nb, _ = blocks.shape
    T = xq.shape[0]
    D = np.zeros((T, M, nb * 8), dtype=np.int64)
    for i in range(M):
        for b in range(nb):
            for j in range(8):
                for l in range(32):
                    byte = int(blocks[i, b, 48 + 32 * (j // 2) + l])
                    nib = (byte >> 4) if (j % 2) else (byte & 15)
                    q5 = nib + 16 * ((int(blocks[i, b, 16 + l]) >> j) & 1)
                    for t in range(T):
                        D[t, i, b * 8 + j] += q5 * int(np.int8(xq[t, b * 8 + j, 4 + l]))
    return D


def test_subdots_brute_force():
    g = np.random.default_rng(17)
    blocks = qmm_synth.q5k_weights(g, 3, 512)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    D, S = oracle.q5k_subdots(blocks, xq)
    assert np.array_equal(D, _brute_force_q5k(blocks, xq))
    _, _, _, qsum = oracle.q8_1_fields(xq)
    assert np.array_equal(S, qsum)


def test_factored_identity_matches_dense():
    g = np.random.default_rng(19)
    blocks = qmm_synth.q5k_weights(g, 5, 1024)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 3, 1024, outlier_frac=0.05))
    W, X = oracle.q5k_dequant(blocks), oracle.q8_1_dequant(xq)
    y = oracle.dense(W, X)
    assert np.all(np.abs(y - oracle.q5k_factored(blocks, xq)) <= 1e-12 * oracle.abs_bound(W, X))


def test_one_hot_activation_returns_weight_column():
    g = np.random.default_rng(23)
    blocks = qmm_synth.q5k_weights(g, 4, 512)
    W = oracle.q5k_dequant(blocks)
    for e in (0, 31, 32, 300, 511):
        q = np.zeros((16, 32), np.int64)
        q[e // 32, e % 32] = 1
        xq = np.stack([_q8_block(0x3C00, q[s]) for s in range(16)]).reshape(1, 16, 40)
        assert np.array_equal(oracle.dense(W, oracle.q8_1_dequant(xq))[0], W[:, e])
        assert np.array_equal(oracle.q5k_factored(blocks, xq)[0], W[:, e])


def test_zero_scales_give_zero():
    g = np.random.default_rng(29)
    blocks = qmm_synth.q5k_weights(g, 3, 512)
    blocks[:, :, 4:16] = 0
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, 2, 512))
    assert not oracle.dense(oracle.q5k_dequant(blocks), oracle.q8_1_dequant(xq)).any()


def test_generator_layout_sentinels():
    g = np.random.default_rng(0)
    blocks = qmm_synth.q5k_weights(g, 64, 2048)
    d, dmin, _, _, _ = oracle.q5k_fields(blocks)
    for v in (d, dmin):
        assert np.all(np.isfinite(v)) and v.min() >= 0
        assert 0.012 < v.mean() < 0.020


@pytest.mark.parametrize("bad", [(1, 1, 175), (2, 177)])
def test_rejects_wrong_block_size(bad):
    with pytest.raises(ValueError):
        oracle.q5k_fields(np.zeros(bad, np.uint8))
