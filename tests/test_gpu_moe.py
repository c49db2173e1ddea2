"""GPU parity for the MoE grouped GEMM, its weighted combine and the SwiGLU glue.

Covers small ragged routings for both formats, the degenerate routings of
the grouped path (top-1 to one expert equals the dense GEMM bit for bit,
token permutations), and the full routed-expert workload (128 experts,
gate||up 1536 x 2048 and down 2048 x 768 Q4_K, T = 512, top-8).
"""
import numpy as np
import pytest

import oracle
import qmm_synth
from _gpu import assert_parity, dev, host, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu

GEN = {"q4k": (qmm_synth.q4k_weights, oracle.q4k_dequant, qmm.QMM_Q4_K),
       "q5k": (qmm_synth.q5k_weights, oracle.q5k_dequant, qmm.QMM_Q5_K),
       "q6k": (qmm_synth.q6k_weights, oracle.q6k_dequant, qmm.QMM_Q6_K)}


def _experts(fmt, E, M, K, g):
    return np.stack([GEN[fmt][0](g, M, K) for _ in range(E)])


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("E,M,K,T,top_k", [(8, 200, 512, 40, 2), (4, 128, 256, 70, 1), (16, 300, 768, 33, 4)])
def test_per_slot_parity(fmt, E, M, K, T, top_k):
    g = qmm_synth.rng(E + M + T)
    w = _experts(fmt, E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    ids, probs = qmm_synth.router(g, T, E, top_k)
    say(f"moe_grouped_mmq {fmt} per-slot", f"E={E} M={M} K={K} T={T} top_k={top_k}")
    y = host(qmm.moe_grouped_mmq(GEN[fmt][2], dev(w), dev(xq), dev(ids)))
    ref, bound = oracle.grouped_blocks(GEN[fmt][1], w, oracle.q8_1_dequant(xq), ids, 1)
    assert_parity(y, ref, bound, "per-slot")


# Larger routings than the cases above (several id batches per wave of the
# route preparation, thousands of slots per call), and the largest expert
# count the route tables hold (512).
@pytest.mark.parametrize("E,T,top_k", [(8, 768, 8), (16, 6145, 1), (32, 1700, 4), (512, 300, 4)])
def test_route_many_slots(E, T, top_k):
    M, K = 40, 256
    g = qmm_synth.rng(E * T + top_k)
    w = _experts("q4k", E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    ids, _ = qmm_synth.router(g, T, E, top_k)
    say("moe_grouped_mmq q4k per-slot (route)", f"E={E} M={M} K={K} T={T} top_k={top_k} slots={T * top_k}")
    y = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(w), dev(xq), dev(ids)))
    ref, bound = oracle.grouped_blocks(oracle.q4k_dequant, w, oracle.q8_1_dequant(xq), ids, 1)
    assert_parity(y, ref, bound, "per-slot")


# The per-slot expert matvec (the path the grouped GEMM replaces): parity
# with the oracle for activation rows per token and per slot, ragged rows,
# and agreement with the grouped GEMM's per-slot output.
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("E,M,K,T,top_k,per_slot_rows", [(8, 200, 512, 40, 2, False), (16, 99, 768, 13, 4, True),
                                                         (128, 512, 2048, 16, 8, False)])
def test_slot_matvec_parity(fmt, E, M, K, T, top_k, per_slot_rows):
    g = qmm_synth.rng(3 * E + M + T)
    w = _experts(fmt, E, M, K, g)
    rows = T * top_k if per_slot_rows else T
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, rows, K))
    ids, _ = qmm_synth.router(g, T, E, top_k)
    say(f"moe_slot_mmvq {fmt}", f"E={E} M={M} K={K} T={T} top_k={top_k} rows={rows}")
    wd, xd, idd = dev(w), dev(xq), dev(ids)
    y = host(qmm.moe_slot_mmvq(GEN[fmt][2], wd, xd, idd))
    ref, bound = oracle.grouped_blocks(GEN[fmt][1], w, oracle.q8_1_dequant(xq), ids, top_k if per_slot_rows else 1)
    assert_parity(y, ref, bound, "slot matvec")
    yg = host(qmm.moe_grouped_mmq(GEN[fmt][2], wd, xd, idd))
    assert_parity(y, yg.astype(np.float64), 2 * bound, "slot matvec vs grouped")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_weighted_slot_rows_parity(fmt):
    E, M, K, T, top_k = 8, 136, 512, 50, 3
    g = qmm_synth.rng(21)
    w = _experts(fmt, E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T * top_k, K))   # one row per slot
    ids, probs = qmm_synth.router(g, T, E, top_k)
    say(f"moe_grouped_mmq {fmt} weighted", f"E={E} M={M} K={K} T={T} top_k={top_k}")
    y = host(qmm.moe_grouped_mmq(GEN[fmt][2], dev(w), dev(xq), dev(ids), dev(probs)))
    ys, bs = oracle.grouped_blocks(GEN[fmt][1], w, oracle.q8_1_dequant(xq), ids, top_k)
    ref = oracle.combine(ys, probs)
    bound = oracle.combine(bs, np.abs(probs))
    assert_parity(y, ref, bound, "weighted")


def test_top1_single_expert_equals_dense_gemm():
    g = qmm_synth.rng(31)
    E, M, K, T = 4, 260, 768, 97
    w = _experts("q4k", E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    ids = np.zeros((T, 1), np.int32)
    say("moe top-1 to expert 0 vs mmq_q4k", f"M={M} K={K} T={T}")
    y_moe = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(w), dev(xq), dev(ids)))
    y_mmq = host(qmm.mmq_q4k(dev(np.ascontiguousarray(w[0])), dev(xq)))
    assert np.array_equal(y_moe.view(np.uint32), y_mmq.view(np.uint32))


def test_token_permutation_permutes_outputs():
    g = qmm_synth.rng(41)
    E, M, K, T, top_k = 8, 128, 512, 60, 2
    w = _experts("q4k", E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    ids, probs = qmm_synth.router(g, T, E, top_k)
    perm = np.random.default_rng(0).permutation(T)
    say("moe permutation", f"E={E} T={T}")
    a = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(w), dev(xq), dev(ids), dev(probs)))
    b = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(w), dev(xq[perm]), dev(ids[perm]), dev(probs[perm])))
    assert np.array_equal(a[perm].view(np.uint32), b.view(np.uint32))


def test_swiglu_glue_properties():
    g = qmm_synth.rng(51)
    R, F = 77, 768
    gu = (g.standard_normal((R, 2 * F)) * 3).astype(np.float32)
    say("swiglu_q8_1", f"R={R} F={F}")
    hq = host(qmm.swiglu_q8_1(dev(gu)))
    h = oracle.swiglu(gu[:, :F], gu[:, F:]).reshape(R, F // 32, 32)
    d16, q, pad, qsum = oracle.q8_1_fields(hq)
    assert not pad.any() and np.array_equal(qsum, q.sum(-1))
    am = np.abs(h).max(-1)
    assert np.all(np.abs(q).max(-1)[am > 0] == 127)
    d = am / 127.0
    assert np.all(np.abs(d16 - d) <= d * 2.0**-10 + 1e-12)          # f16 rounding of d
    err = np.abs(d16[..., None] * q - h)
    assert np.all(err <= d[..., None] * (0.5 + 2.0**-15 + 127 * 2.0**-11) * (1 + 1e-5) + 1e-6 * np.abs(h))


def test_full_routed_ffn_workload():
    """128 experts, T = 512, top-8: gate||up per-slot, then down weighted."""
    wl = qmm_synth.workload(4)
    E, H, F, T, top_k = 128, 2048, 768, 512, 8
    gate_up, down, x, ids, probs = wl["gate_up"], wl["down"], wl["x"], wl["ids"], wl["probs"]
    xq = oracle.quantize_q8_1(x)
    say("moe gate||up per-slot", f"E={E} M={2 * F} K={H} T={T} top_k={top_k}")
    y1 = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(gate_up), dev(xq), dev(ids)))
    ref1, b1 = oracle.grouped_blocks(oracle.q4k_dequant, gate_up, oracle.q8_1_dequant(xq), ids, 1)
    assert_parity(y1, ref1, b1, "gate_up")
    # down projection on an intermediate made by the oracle from its own gate/up
    h = oracle.swiglu(ref1[:, :F], ref1[:, F:]).astype(np.float32)
    hq = oracle.quantize_q8_1(h)
    say("moe down weighted", f"E={E} M={H} K={F} T={T} top_k={top_k}")
    y2 = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), dev(hq), dev(ids), dev(probs)))
    ys, bs = oracle.grouped_blocks(oracle.q4k_dequant, down, oracle.q8_1_dequant(hq), ids, top_k)
    assert_parity(y2, oracle.combine(ys, probs), oracle.combine(bs, np.abs(probs)), "down")
    # determinism of the full call
    y2b = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), dev(hq), dev(ids), dev(probs)))
    assert np.array_equal(y2.view(np.uint32), y2b.view(np.uint32))
