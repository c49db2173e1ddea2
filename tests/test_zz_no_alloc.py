"""The no-allocation GEMM entry point against the workspace entry point.

mmq_q4k_noalloc runs the kernels of mmq_q4k with the library's static device
array as workspace.  Called through the C ABI (ctypes) three times in a row
-- a prefill shape, then a smaller call, then a few-token call that splits K
and so also uses the array for fp32 partial tiles -- each result must equal
mmq_q4k's bit for bit (same kernels, same split factor), and mmq_q4k's
result is itself held to the oracle's tolerance.  A call needing more than
the array holds is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import qmm_synth
from _gpu import assert_parity, dev, host, say

import quantized_matmul_q8_amd as qmm
from quantized_matmul_q8_amd import _lib

pytestmark = pytest.mark.gpu


def _noalloc(w, xq, M, K, T):
    y = torch.full((T, M), float("nan"), dtype=torch.float32, device=w.device)
    st = _lib.LIB.mmq_q4k_noalloc(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(xq.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), M, K, T,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.QMM_OK, _lib.LIB.qmm_status_str(st)
    return y


@pytest.mark.parametrize("M,K,T,seed", [(4096, 4096, 512, 1), (1000, 2048, 70, 2), (4096, 11008, 8, 3)])
def test_noalloc_equals_workspace_call(M, K, T, seed):
    g = qmm_synth.rng(700 + seed)
    w = qmm_synth.q4k_weights(g, M, K)
    xq = oracle.quantize_q8_1(qmm_synth.activations(g, T, K, outlier_frac=0.01))
    need = qmm.workspace_bytes(qmm.QMM_OP_MMQ, M, K, T)
    assert need <= _lib.QMM_STATIC_SCRATCH_BYTES
    say("mmq_q4k_noalloc vs mmq_q4k", f"M={M} K={K} T={T} ws={need}")
    wd, xd = dev(w), dev(xq)
    y_ws = host(qmm.mmq_q4k(wd, xd))
    y_na = host(_noalloc(wd, xd, M, K, T))
    assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32))
    if M * T <= 600_000:    # the oracle on the smaller shapes
        W, X = oracle.q4k_dequant(w), oracle.q8_1_dequant(xq)
        assert_parity(y_na, oracle.dense(W, X), oracle.abs_bound(W, X), "noalloc")


def test_noalloc_two_calls_in_a_row_second_smaller():
    g = qmm_synth.rng(710)
    shapes = [(2048, 4096, 600), (512, 1024, 33)]
    outs = []
    for M, K, T in shapes:
        w = dev(qmm_synth.q4k_weights(g, M, K))
        xq = dev(oracle.quantize_q8_1(qmm_synth.activations(g, T, K)))
        outs.append((w, xq, M, K, T))
    say("mmq_q4k_noalloc twice", shapes)
    ys = [_noalloc(w, xq, M, K, T) for w, xq, M, K, T in outs]     # back to back on one stream
    for (w, xq, M, K, T), y in zip(outs, ys):
        ref = host(qmm.mmq_q4k(w, xq))
        assert np.array_equal(host(y).view(np.uint32), ref.view(np.uint32))


def test_noalloc_refuses_oversize_call():
    say("mmq_q4k_noalloc oversize", "no launch")
    M, K, T = 4096, 4096, 8192
    assert qmm.workspace_bytes(qmm.QMM_OP_MMQ, M, K, T) > _lib.QMM_STATIC_SCRATCH_BYTES
    w = torch.zeros((M, K // 256, 144), dtype=torch.uint8, device="cuda")
    xq = torch.zeros((T, K // 32, 40), dtype=torch.uint8, device="cuda")
    y = torch.zeros((T, M), dtype=torch.float32, device="cuda")
    st = _lib.LIB.mmq_q4k_noalloc(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(xq.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), M, K, T, ctypes.c_void_p(0))
    assert st == _lib.QMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not y.any()
