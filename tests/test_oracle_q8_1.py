"""Pins for the oracle's Q8_1 quantizer (CPU only).

Every expected value here is fixed by IEEE 754 facts, hand-derived fixtures
(tests/golden/q8_1_blocks.txt) or invariants of the quantizer of minfer
ch. 06 "decode MMVQ: dp4a integer dot products", sections 2 and 3.2.
"""
import numpy as np
import pytest

import oracle
from _golden import hexbytes, load, pairs


def _block_from(rec):
    x = np.zeros((1, 32), dtype=np.float32)
    for k, v in pairs(rec.get("x", "")).items():
        x[0, k] = np.float32(v)
    return x


@pytest.mark.parametrize("rec", load("q8_1_blocks.txt"), ids=lambda r: r["name"])
def test_golden_blocks(rec):
    x = _block_from(rec)
    got = oracle.quantize_q8_1(x).reshape(-1).tobytes()
    assert got == hexbytes(rec["bytes"])


def test_f16_cast_is_round_to_nearest_even():
    # IEEE binary16 facts: 1+2^-11 ties to 0x3C00, 1+3*2^-11 ties to 0x3C02,
    # 2^-24 is 0x0001, 0.75*2^-24 rounds to 0x0001, 65504 is 0x7BFF.
    vals = np.array([1 + 2**-11, 1 + 3 * 2**-11, 2**-24, 0.75 * 2**-24, 65504.0], dtype=np.float32)
    bits = vals.astype(np.float16).view(np.uint16).tolist()
    assert bits == [0x3C00, 0x3C02, 0x0001, 0x0001, 0x7BFF]


def test_rint_is_half_even_in_float32():
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5], dtype=np.float32)
    assert np.rint(v).tolist() == [0, 2, 2, -0, -2, -2, 126]


@pytest.mark.parametrize("e", [-30, -20, -8, 0, 3, 9])
def test_power_of_two_grid_is_exact(e):
    # x = k * 2^e with max |x| = 127 * 2^e: d = 2^e, 1/d = 2^-e, q = k exactly.
    k = np.arange(-124, 128, 8, dtype=np.int64)      # 32 values
    k[0] = 127
    x = (k.astype(np.float64) * 2.0**e).astype(np.float32).reshape(1, 32)
    d, q, pad, qsum = oracle.q8_1_fields(oracle.quantize_q8_1(x))
    assert q.reshape(-1).tolist() == k.tolist()
    assert pad[0, 0] == 0 and qsum[0, 0] == k.sum()
    assert d[0, 0] == np.float64(np.float16(np.float32(2.0**e)))


def _random_blocks(n_rows=64, K=1024, seed=123, outliers=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n_rows, K), dtype=np.float32)
    if outliers:
        m = g.random((n_rows, K)) < 0.01
        x = np.where(m, x * np.float32(20), x).astype(np.float32)
    x[0, :32] = 0.0                       # one all-zero block
    x[1, 32:64] = np.float32(1e-30)       # a block of tiny values (d is f16 zero)
    return x


def test_invariants_random_blocks():
    x = _random_blocks()
    xq = oracle.quantize_q8_1(x)
    d16, q, pad, qsum = oracle.q8_1_fields(xq)
    xb = x.reshape(x.shape[0], -1, 32).astype(np.float64)
    am = np.abs(xb).max(axis=-1)
    nz = am > 0
    # stored sum equals the payload sum
    assert np.array_equal(qsum, q.sum(axis=-1))
    # pad is zero
    assert not pad.any()
    # the element reaching max |x| maps to +-127; the clamp never binds
    assert np.all(np.abs(q).max(axis=-1)[nz] == 127)
    assert q.min() >= -127
    # round trip with the float32 d: |x - q d32| <= d32 (1/2 + 2^-15)
    d32 = (am.astype(np.float32) / np.float32(127)).astype(np.float64)
    err = np.abs(xb - q * d32[..., None]).max(axis=-1)
    assert np.all(err <= d32 * (0.5 + 2.0**-15))
    # with the stored f16 d the bound grows by |q| |d32 - d16|
    err16 = np.abs(xb - q * d16[..., None])
    bound16 = d32[..., None] * (0.5 + 2.0**-15) + np.abs(q) * np.abs(d32 - d16)[..., None]
    assert np.all(err16 <= bound16)
    # zero block -> zero bytes
    assert not xq[0, 0].any()


def test_sign_symmetry():
    # rint and the clamp are odd functions: negating x negates q, keeps d.
    x = _random_blocks(outliers=False)
    a = oracle.q8_1_fields(oracle.quantize_q8_1(x))
    b = oracle.q8_1_fields(oracle.quantize_q8_1(-x))
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], -b[1])


def test_scale_invariance_by_powers_of_two():
    # Scaling x by 2^k scales d by 2^k and leaves q unchanged (all steps exact
    # under power-of-two scaling away from under/overflow).
    x = _random_blocks(outliers=False)
    a = oracle.q8_1_fields(oracle.quantize_q8_1(x))
    b = oracle.q8_1_fields(oracle.quantize_q8_1((x * np.float32(8)).astype(np.float32)))
    assert np.array_equal(a[1], b[1])
    big = a[0] > 2**-10                   # stay clear of f16 subnormals
    assert np.array_equal(a[0][big] * 8, b[0][big])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize_q8_1(np.zeros((1, 33), np.float32))
    with pytest.raises(TypeError):
        oracle.quantize_q8_1(np.zeros((1, 32), np.float64))
