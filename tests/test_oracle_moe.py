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


# ---------------------------------------------------------------------------
# grouped_blocks (the reference of every grouped GPU test) and abs_bound (the
# tolerance scale of every parity assertion), pinned against plain loops.
# ---------------------------------------------------------------------------
def _fsum_dot(a, b):
    import math
    return math.fsum(float(u) * float(v) for u, v in zip(a, b))


def _slot_loop(W, X, ids, rows_per_token):
    """y_slot and bound by the definition: slot s = t*top_k + k multiplies
    expert ids[t, k] with activation row t (one row per token) or s (one row
    per slot); exactly rounded sums (math.fsum), no BLAS."""
    T, top_k = ids.shape
    M = W.shape[1]
    y = np.zeros((T * top_k, M))
    b = np.zeros((T * top_k, M))
    for t in range(T):
        for k in range(top_k):
            s = t * top_k + k
            row = t if rows_per_token == 1 else s
            e = int(ids[t, k])
            for i in range(M):
                y[s, i] = _fsum_dot(W[e, i], X[row])
                b[s, i] = _fsum_dot(np.abs(W[e, i]), np.abs(X[row]))
    return y, b


@pytest.mark.parametrize("per_slot_rows", [False, True])
def test_grouped_blocks_matches_definition_loop(per_slot_rows):
    # expert 3 of 5 receives no slot; tokens route to 2 experts each
    g, blocks, W = _experts(E=5, M=3, K=256, seed=11)
    T, top_k = 4, 2
    ids = np.array([[0, 4], [4, 1], [2, 0], [1, 4]], dtype=np.int32)
    rows = T * top_k if per_slot_rows else T
    X = oracle.q8_1_dequant(oracle.quantize_q8_1(qmm_synth.activations(g, rows, 256)))
    r = top_k if per_slot_rows else 1
    y, bound = oracle.grouped_blocks(oracle.q4k_dequant, blocks, X, ids, r)
    y_ref, b_ref = _slot_loop(W, X, ids, r)
    scale = np.abs(W).max() * np.abs(X).max() * 256
    assert np.all(np.abs(y - y_ref) <= 1e-13 * scale)
    assert np.all(np.abs(bound - b_ref) <= 1e-13 * b_ref + 1e-300)
    assert np.all(bound >= np.abs(y) * (1 - 1e-13))


@pytest.mark.parametrize("per_slot_rows", [False, True])
def test_grouped_blocks_equals_grouped_on_dequantized_experts(per_slot_rows):
    g, blocks, W = _experts(E=6, M=16, K=512, seed=12)
    T, top_k = 9, 3
    ids, _ = qmm_synth.router(g, T, 5, top_k)      # expert 5 never routed
    rows = T * top_k if per_slot_rows else T
    X = oracle.q8_1_dequant(oracle.quantize_q8_1(qmm_synth.activations(g, rows, 512)))
    r = top_k if per_slot_rows else 1
    y, bound = oracle.grouped_blocks(oracle.q4k_dequant, blocks, X, ids, r)
    assert np.array_equal(y, oracle.grouped(W, X, ids, r))
    # bound[s] = |x_row| . |W_e|^T, the per-slot abs_bound
    T_, k_ = ids.shape
    for t in range(T_):
        for k in range(k_):
            s = t * k_ + k
            row = t if r == 1 else s
            assert np.array_equal(bound[s], oracle.abs_bound(W[ids[t, k]], X[row:row + 1])[0])


def test_grouped_blocks_expert_subset_fills_only_those_slots():
    g, blocks, W = _experts(E=4, M=8, K=256, seed=13)
    T, top_k = 10, 2
    ids, _ = qmm_synth.router(g, T, 4, top_k)
    X = oracle.q8_1_dequant(oracle.quantize_q8_1(qmm_synth.activations(g, T, 256)))
    full, bfull = oracle.grouped_blocks(oracle.q4k_dequant, blocks, X, ids, 1)
    part, bpart = oracle.grouped_blocks(oracle.q4k_dequant, blocks, X, ids, 1, experts=[1, 3])
    sel = np.isin(ids.ravel(), [1, 3])
    assert np.array_equal(part[sel], full[sel]) and np.array_equal(bpart[sel], bfull[sel])
    assert not part[~sel].any() and not bpart[~sel].any()


def test_abs_bound_brute_force():
    # signs mixed on both sides; the bound is sum_k |w_ik| |x_tk|, never the
    # magnitude of the signed sum
    W = np.array([[1.0, -2.0, 0.5], [-0.25, 0.0, 3.0]])
    X = np.array([[2.0, 1.0, -4.0], [-1.0, -1.0, -1.0], [0.0, 0.0, 0.0]])
    b = oracle.abs_bound(W, X)
    expect = [[1 * 2 + 2 * 1 + 0.5 * 4, 0.25 * 2 + 0 + 3 * 4],
              [1 + 2 + 0.5, 0.25 + 0 + 3],
              [0.0, 0.0]]
    assert b.shape == (3, 2) and np.array_equal(b, np.array(expect))
    g = np.random.default_rng(5)
    W = g.standard_normal((3, 7))
    X = g.standard_normal((4, 7))
    b = oracle.abs_bound(W, X)
    for t in range(4):
        for i in range(3):
            assert abs(b[t, i] - _fsum_dot(np.abs(W[i]), np.abs(X[t]))) <= 1e-14 * b[t, i]
