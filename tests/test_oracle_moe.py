"""Pins for the oracle's MoE grouping, grouped products and combine (CPU only).

Anchors: brute force on small routings, the degenerate cases of the grouped
path described in "Prefill Gap Closure Plan -- ZINC CUDA vs llama.cpp", lever
T2 (top-1 routing to one expert is a dense product; permuting tokens permutes
outputs), and closed forms for the combine and the SwiGLU glue.
"""
import numpy as np
import pytest

import oracle
import qmm_synth


def test_route_buckets_small_brute_force():
    ids = np.array([[2, 0], [2, 1], [0, 2]], dtype=np.int32)
    counts, offsets, bucket = oracle.route_buckets(ids, 4)
    assert counts.tolist() == [2, 1, 3, 0]
    assert offsets.tolist() == [0, 2, 3, 6, 6]
    # slots: 0:(t0,e2) 1:(t0,e0) 2:(t1,e2) 3:(t1,e1) 4:(t2,e0) 5:(t2,e2)
    assert bucket.tolist() == [1, 4, 3, 0, 2, 5]


def test_route_buckets_random_properties():
    g = qmm_synth.rng(9)
    ids, _ = qmm_synth.router(g, 300, 32, 4)
    counts, offsets, bucket = oracle.route_buckets(ids, 32)
    assert counts.sum() == ids.size
    assert sorted(bucket.tolist()) == list(range(ids.size))
    flat = ids.ravel()
    for e in range(32):
        sl = bucket[offsets[e]:offsets[e + 1]]
        assert np.all(flat[sl] == e) and np.all(np.diff(sl) > 0)


def test_route_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.route_buckets(np.array([[5]]), 4)


def test_router_generator():
    g = qmm_synth.rng(4)
    ids, probs = qmm_synth.router(g, 64, 128, 8)
    assert ids.shape == (64, 8) and probs.shape == (64, 8)
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.all(np.diff(probs.astype(np.float64), axis=1) <= 0)
    assert np.all(probs.sum(axis=1) < 1.0)


def _experts(E=4, M=8, K=256, seed=2):
    g = qmm_synth.rng(seed)
    blocks = np.stack([qmm_synth.q4k_weights(g, M, K) for _ in range(E)])
    W = np.stack([oracle.q4k_dequant(b) for b in blocks])
    return g, blocks, W


def test_top1_single_expert_is_dense():
    g, blocks, W = _experts()
    X = oracle.q8_1_dequant(oracle.quantize_q8_1(qmm_synth.activations(g, 6, 256)))
    ids = np.zeros((6, 1), np.int32)
    ys = oracle.grouped(W, X, ids, rows_per_token=1)
    assert np.array_equal(ys, oracle.dense(W[0], X))


def test_grouped_matches_per_slot_loop_and_permutation():
    g, blocks, W = _experts()
    T, k = 7, 2
    X = oracle.q8_1_dequant(oracle.quantize_q8_1(qmm_synth.activations(g, T, 256)))
    ids, probs = qmm_synth.router(g, T, 4, k)
    ys = oracle.grouped(W, X, ids, rows_per_token=1)
    for t in range(T):
        for kk in range(k):
            assert np.allclose(ys[t * k + kk], W[ids[t, kk]] @ X[t], rtol=1e-14, atol=1e-14)
    perm = np.random.default_rng(1).permutation(T)
    ys_p = oracle.grouped(W, X[perm], ids[perm], rows_per_token=1).reshape(T, k, -1)
    assert np.allclose(ys_p, ys.reshape(T, k, -1)[perm], rtol=1e-14, atol=1e-14)
    # one activation row per slot (down projection mode)
    Xs = np.repeat(X, k, axis=0)
    assert np.allclose(oracle.grouped(W, Xs, ids, rows_per_token=k), ys, rtol=1e-14, atol=1e-14)


def test_combine_closed_forms():
    ys = np.arange(2 * 3 * 4, dtype=np.float64).reshape(6, 4)
    p = np.array([[1.0, 0.0, 0.0], [0.5, 0.25, 0.25]])
    y = oracle.combine(ys, p)
    assert np.array_equal(y[0], ys[0])
    assert np.array_equal(y[1], 0.5 * ys[3] + 0.25 * ys[4] + 0.25 * ys[5])


def test_swiglu_closed_forms():
    assert oracle.swiglu(np.array([0.0]), np.array([3.0]))[0] == 0.0
    g = np.array([2.0])
    assert np.isclose(oracle.swiglu(g, np.array([1.0]))[0], 2.0 / (1.0 + np.exp(-2.0)), rtol=1e-15)
    assert np.isclose(oracle.swiglu(np.array([50.0]), np.array([2.0]))[0], 100.0, rtol=1e-15)
