"""GPU parity for the MoE grouped GEMM, its weighted combine and the SwiGLU glue.

Covers small ragged routings for both formats, the degenerate routings of
the grouped path (top-1 to one expert against the dense GEMM,
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
# route preparation, thousands of slots per call; above 8192 slots a wave's
# slots take more than one batch and are ranked in the second pass), and the
# largest expert count the route tables hold (512).
@pytest.mark.parametrize("E,T,top_k", [(8, 768, 8), (16, 6145, 1), (32, 1700, 4), (512, 300, 4), (8, 2100, 4)])
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


@pytest.mark.parametrize("K", [1024, 768])
def test_top1_single_expert_matches_dense_gemm(K):
    # Top-1 routing of every token to expert 0 is the dense product with that
    # expert's weights.  The grouped Q4_K tiles take every super-block of a
    # row in one wave while the dense GEMM sums two K halves, so the fp32
    # sums run in different orders: both are held to the oracle, and to each
    # other within twice the tolerance.
    g = qmm_synth.rng(31)
    E, M, T = 4, 260, 97
    w = _experts("q4k", E, M, K, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    ids = np.zeros((T, 1), np.int32)
    say("moe top-1 to expert 0 vs mmq_q4k", f"M={M} K={K} T={T}")
    y_moe = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(w), dev(xq), dev(ids)))
    y_mmq = host(qmm.mmq_q4k(dev(np.ascontiguousarray(w[0])), dev(xq)))
    W, X = oracle.q4k_dequant(w[0]), oracle.q8_1_dequant(xq)
    ref, bound = oracle.dense(W, X), oracle.abs_bound(W, X)
    assert_parity(y_moe, ref, bound, "grouped top-1")
    assert_parity(y_mmq, ref, bound, "dense")
    assert_parity(y_moe, y_mmq.astype(np.float64), 2 * bound, "grouped vs dense")


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_routed_call_reuses_route_tables(fmt):
    # a per-slot call (gate||up shape) prepares the routing in ws; the weighted
    # call that follows on the same ws with reuse_routing (other M and K, one
    # activation row per slot) must equal the same call routed afresh
    E, T, top_k, H, F = 16, 70, 4, 512, 256
    g = qmm_synth.rng(53)
    w_gu = _experts(fmt, E, 2 * F, H, g)
    w_dn = _experts(fmt, E, H, F, g)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, H))
    hq = oracle.quantize_q8_1(qmm_synth.activations(g, T * top_k, F))
    ids, probs = qmm_synth.router(g, T, E, top_k)
    need = max(qmm.workspace_bytes(qmm.QMM_OP_MOE_SLOTS, 2 * F, H, T, E, top_k),
               qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k))
    ws = qmm.workspace(need, dev(ids).device)
    say(f"moe_grouped_mmq_routed {fmt}", f"E={E} T={T} top_k={top_k} H={H} F={F}")
    d_ids, d_probs, d_hq, d_wdn = dev(ids), dev(probs), dev(hq), dev(w_dn)
    qmm.moe_grouped_mmq(GEN[fmt][2], dev(w_gu), dev(xq), d_ids, ws=ws)
    y_routed = host(qmm.moe_grouped_mmq(GEN[fmt][2], d_wdn, d_hq, d_ids, d_probs, ws=ws, reuse_routing=True))
    y_fresh = host(qmm.moe_grouped_mmq(GEN[fmt][2], d_wdn, d_hq, d_ids, d_probs))
    assert np.array_equal(y_routed.view(np.uint32), y_fresh.view(np.uint32))
    ys, bs = oracle.grouped_blocks(GEN[fmt][1], w_dn, oracle.q8_1_dequant(hq), ids, top_k)
    assert_parity(y_routed, oracle.combine(ys, probs), oracle.combine(bs, np.abs(probs)), "routed weighted")


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


def _q8_1_error_bound(hq):
    """Per element bound of |x - d16*q| for a Q8_1 block of d16, from the
    quantizer's round-trip pin: d32*(1/2 + 2^-15) + |q|*|d32 - d16|, with
    d32 within one f16 rounding of d16 (relative 2^-11, absolute 2^-25)."""
    d16, q, _, _ = oracle.q8_1_fields(hq)
    d32_hi = d16 * (1 + 2.0**-10) + 2.0**-25
    dd = d16 * 2.0**-10 + 2.0**-25
    return (d32_hi * (0.5 + 2.0**-15))[..., None] + np.abs(q) * dd[..., None]


def test_full_routed_ffn_gpu_chain():
    """128 experts, T = 512, top-8, the whole routed FFN on the GPU (quantize,
    grouped gate||up, SwiGLU -> Q8_1, grouped down with the routing weights,
    reusing the gate||up call's route tables)
    against the oracle chain, with the tolerance carried through the glue:

      |y2_gpu - y2_ora| <= sum_k p_k sum_j |W_down| |x_gpu - x_ora|  +  1e-4 sum_k p_k sum_j |W_down| |x_gpu|

    (triangle inequality: the second term is the grouped GEMM's own parity
    bound on the GPU intermediate, the first the exact effect of the
    intermediate's difference), where x_gpu, x_ora are the dequantized
    SwiGLU activations of the two chains, and |x_gpu - x_ora| is itself held
    to the bound of the glue: the gate||up parity error carried through
    SwiGLU plus both quantization errors."""
    wl = qmm_synth.workload(4)
    E, H, F, T, top_k = 128, 2048, 768, 512, 8
    gate_up, down, x, ids, probs = wl["gate_up"], wl["down"], wl["x"], wl["ids"], wl["probs"]
    say("moe routed FFN GPU chain", f"E={E} H={H} F={F} T={T} top_k={top_k}")
    xq_gpu = qmm.q8_1_quantize(dev(x))
    xq = oracle.quantize_q8_1(x)
    assert np.array_equal(host(xq_gpu), xq)
    # one workspace for both calls; the down call reuses the gate||up routing
    ws = qmm.workspace(max(qmm.workspace_bytes(qmm.QMM_OP_MOE_SLOTS, 2 * F, H, T, E, top_k),
                           qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k)), xq_gpu.device)
    d_ids = dev(ids)
    y1_d = qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(gate_up), xq_gpu, d_ids, ws=ws)
    hq_d = qmm.swiglu_q8_1(y1_d)
    y2 = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), hq_d, d_ids, dev(probs), ws=ws, reuse_routing=True))
    y1, hq_gpu = host(y1_d), host(hq_d)
    # step 1: gate||up parity
    ref1, b1 = oracle.grouped_blocks(oracle.q4k_dequant, gate_up, oracle.q8_1_dequant(xq), ids, 1)
    assert_parity(y1, ref1, b1, "gate_up")
    # step 2: the glue.  SwiGLU h = silu(g) u; |silu'| <= 1.1, so an error
    # e_g in g and e_u in u move h by at most 1.1 e_g (|u| + e_u) + |silu(g)| e_u,
    # plus the fp32 evaluation (a few ulps: 2^-20 |h| with margin)
    g_r, u_r = ref1[:, :F], ref1[:, F:]
    e_g, e_u = 1e-4 * b1[:, :F], 1e-4 * b1[:, F:]
    h_ora = oracle.swiglu(g_r, u_r)
    silu = oracle.swiglu(g_r, np.ones_like(g_r))
    dh = 1.1 * e_g * (np.abs(u_r) + e_u) + np.abs(silu) * e_u + 2.0**-20 * np.abs(h_ora)
    hq_ora = oracle.quantize_q8_1(h_ora.astype(np.float32))
    x_gpu = oracle.q8_1_dequant(hq_gpu)
    x_ora = oracle.q8_1_dequant(hq_ora)
    qe = _q8_1_error_bound(hq_gpu).reshape(T * top_k, F) + _q8_1_error_bound(hq_ora).reshape(T * top_k, F)
    dx = np.abs(x_gpu - x_ora)
    assert np.all(dx <= (dh + qe) * (1 + 1e-9) + 1e-30), "SwiGLU glue outside its carried bound"
    # step 3: down + ordered combine against the oracle chain
    ys_g, bs_g = oracle.grouped_blocks(oracle.q4k_dequant, down, x_gpu, ids, top_k)
    ys_o, _ = oracle.grouped_blocks(oracle.q4k_dequant, down, x_ora, ids, top_k)
    carried, _ = oracle.grouped_blocks(lambda b: np.abs(oracle.q4k_dequant(b)), down, dx, ids, top_k)
    pa = np.abs(probs)
    y2_g, y2_o = oracle.combine(ys_g, probs), oracle.combine(ys_o, probs)
    tol = oracle.combine(carried, pa) + 1e-4 * oracle.combine(bs_g, pa)
    # the last step on the GPU's own intermediate (exact reference) ...
    assert_parity(y2, y2_g, oracle.combine(bs_g, pa), "down on the GPU intermediate")
    # ... and the whole chain against the oracle's
    err = np.abs(y2.astype(np.float64) - y2_o)
    bad = err > tol * (1 + 1e-9)
    assert not bad.any(), f"{int(bad.sum())} outputs outside the carried tolerance (max excess {np.max(err - tol):.3e})"
    # the fused gate||up + SwiGLU call gives the same bytes, and the down call
    # on its route tables the same output
    ws_f = qmm.workspace(ws.numel(), xq_gpu.device)
    hq_f = qmm.moe_grouped_swiglu(qmm.QMM_Q4_K, dev(gate_up), xq_gpu, d_ids, ws=ws_f)
    assert np.array_equal(host(hq_f), hq_gpu), "fused SwiGLU bytes differ from gate||up + swiglu_q8_1"
    y2f = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), hq_f, d_ids, dev(probs), ws=ws_f, reuse_routing=True))
    assert np.array_equal(y2f.view(np.uint32), y2.view(np.uint32))
    # determinism of the full chain
    y2b = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), qmm.swiglu_q8_1(
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(gate_up), xq_gpu, dev(ids))), dev(ids), dev(probs)))
    assert np.array_equal(y2.view(np.uint32), y2b.view(np.uint32))


# The grouped gate||up call with SwiGLU -> Q8_1 fused into its epilogue: the
# bytes of moe_grouped_mmq (per slot) followed by swiglu_q8_1, for both
# formats it takes, activation rows per token and per slot, ragged routings
# (experts with no slot, partial column tiles), two to four 128-row tiles per
# half; the down call then reuses the route tables it left.
@pytest.mark.parametrize("fmt", ["q4k", "q5k"])
@pytest.mark.parametrize("E,F,H,T,top_k,per_slot_rows", [(16, 256, 512, 70, 4, False), (8, 512, 768, 33, 2, True),
                                                         (40, 256, 256, 5, 3, False)])
def test_fused_swiglu_matches_unfused(fmt, E, F, H, T, top_k, per_slot_rows):
    g = qmm_synth.rng(E + F + T)
    gate_up = _experts(fmt, E, 2 * F, H, g)
    down = _experts("q4k", E, H, F, g)
    rows = T * top_k if per_slot_rows else T
    xq = dev(oracle.quantize_q8_1(qmm_synth.activations(g, rows, H)))
    ids, probs = qmm_synth.router(g, T, E, top_k)
    d_ids = dev(ids)
    say(f"moe_grouped_swiglu {fmt}", f"E={E} F={F} H={H} T={T} top_k={top_k} per_slot_rows={per_slot_rows}")
    ws = qmm.workspace(max(qmm.workspace_bytes(qmm.QMM_OP_MOE_SLOTS, 2 * F, H, T, E, top_k),
                           qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k)), xq.device)
    hq_f = qmm.moe_grouped_swiglu(GEN[fmt][2], dev(gate_up), xq, d_ids, ws=ws)
    y_f = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), hq_f, d_ids, dev(probs), ws=ws, reuse_routing=True))
    y1 = qmm.moe_grouped_mmq(GEN[fmt][2], dev(gate_up), xq, d_ids)
    hq_u = host(qmm.swiglu_q8_1(y1))
    assert np.array_equal(host(hq_f), hq_u)
    y_u = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dev(down), dev(hq_u), d_ids, dev(probs)))
    assert np.array_equal(y_f.view(np.uint32), y_u.view(np.uint32))


# The whole routed FFN layer in one call (the gate||up epilogue writing the down
# product's chunks itself): bit-identical to the fused SwiGLU call followed by
# the weighted routed down call, for each down format, and at the full layer.
@pytest.mark.parametrize("fmt_dn", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("E,F,H,T,top_k", [(16, 256, 512, 70, 4), (40, 512, 256, 5, 3)])
def test_moe_ffn_matches_two_calls(fmt_dn, E, F, H, T, top_k):
    g = qmm_synth.rng(E + F + T + 1)
    gate_up = _experts("q4k", E, 2 * F, H, g)
    down = _experts(fmt_dn, E, H, F, g)
    xq = dev(oracle.quantize_q8_1(qmm_synth.activations(g, T, H)))
    ids, probs = qmm_synth.router(g, T, E, top_k)
    d_ids, d_probs = dev(ids), dev(probs)
    say(f"moe_ffn q4k/{fmt_dn}", f"E={E} F={F} H={H} T={T} top_k={top_k}")
    y = host(qmm.moe_ffn(qmm.QMM_Q4_K, dev(gate_up), GEN[fmt_dn][2], dev(down), xq, d_ids, d_probs))
    ws = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k), xq.device)
    hq = qmm.moe_grouped_swiglu(qmm.QMM_Q4_K, dev(gate_up), xq, d_ids, ws=ws)
    y2 = host(qmm.moe_grouped_mmq(GEN[fmt_dn][2], dev(down), hq, d_ids, d_probs, ws=ws, reuse_routing=True))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_moe_ffn_full_layer():
    wl = qmm_synth.workload(4)
    E, H, F, T, top_k = 128, 2048, 768, 512, 8
    say("moe_ffn full layer", f"E={E} H={H} F={F} T={T} top_k={top_k}")
    xq = qmm.q8_1_quantize(dev(wl["x"]))
    d_ids, d_probs = dev(wl["ids"]), dev(wl["probs"])
    gate_up, down = dev(wl["gate_up"]), dev(wl["down"])
    y = host(qmm.moe_ffn(qmm.QMM_Q4_K, gate_up, qmm.QMM_Q4_K, down, xq, d_ids, d_probs))
    hq = qmm.swiglu_q8_1(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, gate_up, xq, d_ids))
    y2 = host(qmm.moe_grouped_mmq(qmm.QMM_Q4_K, down, hq, d_ids, d_probs))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def _near_half(v, ulps):
    """fp32 value v within `ulps` of a rounding tie n + 1/2."""
    v = np.asarray(v, np.float32)
    frac = np.abs(v.astype(np.float64) - np.floor(v.astype(np.float64)) - 0.5)
    return frac <= ulps * np.spacing(np.abs(v)).astype(np.float64)


def test_swiglu_bytes_against_oracle_quantizer():
    """swiglu_q8_1 bytes against the oracle's quantizer applied to an fp32
    SwiGLU computed on the host.  The two fp32 SwiGLUs may differ by an ulp
    (exp is not correctly rounded on either side), so a byte may differ only
    at a rounding boundary: a value q may differ by one where the oracle's
    fp32 product x * (1/d) lies within 8 ulps of a tie, and a block's f16 d
    by one f16 ulp where the fp32 d lies within 8 ulps of an f16 tie."""
    g = qmm_synth.rng(52)
    R, F = 300, 768
    gu = (g.standard_normal((R, 2 * F)) * 3).astype(np.float32)
    say("swiglu_q8_1 bytes", f"R={R} F={F}")
    hq = host(qmm.swiglu_q8_1(dev(gu)))
    gt, ut = gu[:, :F], gu[:, F:]
    with np.errstate(over="ignore"):
        h32 = (gt / (np.float32(1) + np.exp(-gt)) * ut).astype(np.float32)
    ref = oracle.quantize_q8_1(h32)
    d_g, q_g, pad_g, s_g = oracle.q8_1_fields(hq)
    d_o, q_o, _, _ = oracle.q8_1_fields(ref)
    assert not pad_g.any() and np.array_equal(s_g, q_g.sum(-1))
    # the oracle's fp32 intermediates, to locate rounding boundaries
    hb = h32.reshape(R, F // 32, 32)
    d32 = (np.abs(hb).max(-1) / np.float32(127)).astype(np.float32)
    di = np.where(d32 >= np.float32(2.0**-126), (np.float32(1) / d32).astype(np.float32), np.float32(0))
    v = (hb * di[..., None]).astype(np.float32)
    dq = q_g.astype(np.int64) - q_o.astype(np.int64)
    ok_q = (dq == 0) | ((np.abs(dq) == 1) & _near_half(v, 8))
    dd_blocks = d_g != d_o
    # a block whose f16 d differs: d32 must sit at an f16 tie; its q may then differ by one anywhere
    d16_tie = np.abs(d32.astype(np.float64) - (d_g + d_o) / 2) <= 8 * np.spacing(d32).astype(np.float64)
    assert np.all(~dd_blocks | d16_tie), "f16 scale differs away from a rounding tie"
    ok = ok_q | (dd_blocks[..., None] & (np.abs(dq) <= 1))
    assert ok.all(), f"{int((~ok).sum())} values differ away from a rounding boundary"
    n_diff = int((dq != 0).sum())
    say("  bytes differing at rounding boundaries:", n_diff, "of", dq.size)
    assert n_diff <= dq.size // 1000
