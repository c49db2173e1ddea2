"""Argument checks of the Python binding that need device tensors, and the
per-stream GEMM workspace.

The C ABI cannot see buffer sizes, so the binding must reject a caller's
output tensor of the wrong shape before anything is enqueued (these cases
launch no kernel).  The cached GEMM workspace holds a call's queue counters
and repacked activations; calls on different streams must not share it.
"""
import numpy as np
import pytest
import torch

import oracle
import qmm_synth
from _gpu import DEV, dev, host, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu


def _f32(*shape):
    return torch.empty(shape, dtype=torch.float32, device=DEV)


def _u8(*shape):
    return torch.empty(shape, dtype=torch.uint8, device=DEV)


def test_out_shape_rejected_everywhere():
    say("binding out-shape checks", "no kernel launches")
    M, K, T = 64, 256, 3
    w4 = _u8(M, 1, 144)
    w6 = _u8(M, 1, 210)
    xq = _u8(T, K // 32, 40)
    x = _f32(T, K)
    with pytest.raises(ValueError):
        qmm.q8_1_quantize(x, out=_u8(T + 1, K // 32, 40))           # too many rows
    with pytest.raises(ValueError):
        qmm.q8_1_quantize(x, out=_u8(T - 1, K // 32, 40))           # too few rows
    for fn, w in ((qmm.mmvq_q4k, w4), (qmm.mmvq_q6k, w6), (qmm.mmq_q4k, w4), (qmm.mmq_q6k, w6)):
        for bad in ((T, M - 1), (T - 1, M), (T * M,)):
            with pytest.raises(ValueError):
                fn(w, xq, out=_f32(*bad))
    for fn, w in ((qmm.mmq_q4k_f32, w4), (qmm.mmq_q6k_f32, w6)):
        with pytest.raises(ValueError):
            fn(w, x, out=_f32(T, M + 4))
    E, top_k = 4, 2
    we = _u8(E, M, 1, 144)
    ids = torch.zeros((T, top_k), dtype=torch.int32, device=DEV)
    p = torch.zeros((T, top_k), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, we, xq, ids, out=_f32(T, M))              # per slot: T*top_k rows
    with pytest.raises(ValueError):
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, we, xq, ids, p, out=_f32(T * top_k, M))   # weighted: T rows
    with pytest.raises(ValueError):
        qmm.moe_slot_mmvq(qmm.QMM_Q4_K, we, xq, ids, out=_f32(T * top_k - 1, M))


def test_swiglu_rejects_odd_and_ragged_widths():
    say("binding swiglu width checks", "no kernel launches")
    with pytest.raises(ValueError):
        qmm.swiglu_q8_1(_f32(4, 65))          # odd: no gate/up split
    with pytest.raises(ValueError):
        qmm.swiglu_q8_1(_f32(4, 96))          # F = 48 is not a block multiple
    with pytest.raises(ValueError):
        qmm.swiglu_q8_1(_f32(4, 128), out=_u8(5, 2, 40))


def test_workspace_per_stream_and_concurrent_calls():
    """Two GEMMs enqueued on two streams at once, each with the cached
    workspace: results equal the same calls run one after the other."""
    g = qmm_synth.rng(61)
    M, K, T = 1024, 2048, 200
    wa, wb = qmm_synth.q4k_weights(g, M, K), qmm_synth.q4k_weights(g, M, K)
    xa = oracle.quantize_q8_1(qmm_synth.activations(g, T, K))
    xb = oracle.quantize_q8_1(qmm_synth.activations(g, T + 37, K))
    wa_d, wb_d, xa_d, xb_d = dev(wa), dev(wb), dev(xa), dev(xb)
    say("mmq_q4k on two streams", f"M={M} K={K} T={T},{T + 37}")
    ya_ref = host(qmm.mmq_q4k(wa_d, xa_d))
    yb_ref = host(qmm.mmq_q4k(wb_d, xb_d))
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = qmm.mmq_q4k(wa_d, xa_d)
        with torch.cuda.stream(s2):
            yb = qmm.mmq_q4k(wb_d, xb_d)
        torch.cuda.synchronize()
        assert np.array_equal(ya.cpu().numpy().view(np.uint32), ya_ref.view(np.uint32))
        assert np.array_equal(yb.cpu().numpy().view(np.uint32), yb_ref.view(np.uint32))
    keys = [k for k in qmm._MMQ_WS if k[1] in (s1.cuda_stream, s2.cuda_stream)]
    assert len(keys) == 2
