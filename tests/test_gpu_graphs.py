"""HIP graph capture of the hot path: every replay must give the eager result.

The entry points only enqueue kernels (no allocation, no memset: the GEMM and
MoE calls zero their own queue counters in the kernel that precedes the GEMM),
so a caller can capture them.  Each case captures one pass into a torch CUDA
graph on a side stream, then replays it several times with the program's own
eager work and synchronisations between the replays, and compares every
replay bit for bit with an eager run of the same calls on the same inputs; the
inputs are changed in place between replays, so each replay must read them
afresh.  The results are deterministic, so equality is exact.
"""
import numpy as np
import pytest
import torch

import qmm_synth
from _gpu import DEV, dev, say

import quantized_matmul_q8_amd as qmm

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        fn()                     # warm-up on the capture stream
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _check_replays(run, outs, change_inputs, what):
    """run(): the captured calls writing `outs`; replays against fresh eager runs."""
    g = _capture(run)
    for r in range(REPLAYS):
        change_inputs(r)
        torch.cuda.synchronize()
        run()                                    # eager, on the current stream
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan") if o.dtype == torch.float32 else 0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"{what}: replay {r}, output {i} differs from the eager result"
        # unrelated eager work between replays
        torch.cuda.synchronize()
        (torch.randn(1024, device=DEV) * 2).sum().item()


def test_decode_step_graph():
    g = qmm_synth.rng(11)
    M, K = 1024, 11008
    w4, w6 = dev(qmm_synth.q4k_weights(g, M, K)), dev(qmm_synth.q6k_weights(g, M, K))
    x = dev(qmm_synth.activations(g, 1, K))
    xq = torch.empty((1, K // 32, 40), dtype=torch.uint8, device=DEV)
    y4, y6 = (torch.empty((1, M), dtype=torch.float32, device=DEV) for _ in range(2))
    y4s = torch.empty_like(y4)
    say("graph: q8_1_quantize + mmvq_pair + mmvq_q4k", f"M={M} K={K}")

    def run():
        qmm.q8_1_quantize(x, out=xq)
        qmm.mmvq_pair(qmm.QMM_Q6_K, w6, qmm.QMM_Q4_K, w4, xq, out_a=y6, out_b=y4)
        qmm.mmvq_q4k(w4, xq, out=y4s)

    def change(r):
        x.mul_(1.5 if r % 2 else -0.75)

    _check_replays(run, [y4, y6, y4s], change, "decode step")
    assert torch.equal(y4, y4s)


@pytest.mark.parametrize("M,K,T", [(4096, 1024, 512), (1024, 2048, 16)])
def test_gemm_graph(M, K, T):
    # 256 tiles (each tile's whole K loop in one workgroup) and a split-K call
    # (arrival counters zeroed by the repack of every replay)
    g = qmm_synth.rng(M + T)
    w = dev(qmm_synth.q4k_weights(g, M, K))
    x = dev(qmm_synth.activations(g, T, K))
    xq = torch.empty((T, K // 32, 40), dtype=torch.uint8, device=DEV)
    y, yf = (torch.empty((T, M), dtype=torch.float32, device=DEV) for _ in range(2))
    ws = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MMQ, M, K, T), DEV)
    ws2 = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MMQ, M, K, T), DEV)
    say("graph: q8_1_quantize + mmq_q4k + mmq_q4k_f32", f"M={M} K={K} T={T}")

    def run():
        qmm.q8_1_quantize(x, out=xq)
        qmm.mmq_q4k(w, xq, out=y, ws=ws)
        qmm.mmq_q4k_f32(w, x, out=yf, ws=ws2)

    def change(r):
        x.mul_(0.5 if r % 2 else -2.0)

    _check_replays(run, [y, yf], change, f"gemm {M}x{K} T={T}")
    assert torch.equal(y, yf)


def test_routed_ffn_graph():
    E, H, F, T, top_k = 16, 512, 256, 96, 4
    g = qmm_synth.rng(21)
    gate_up = dev(np.stack([qmm_synth.q4k_weights(g, 2 * F, H) for _ in range(E)]))
    down = dev(np.stack([qmm_synth.q4k_weights(g, H, F) for _ in range(E)]))
    x = dev(qmm_synth.activations(g, T, H))
    ids_h, probs_h = qmm_synth.router(g, T, E, top_k)
    ids, probs = dev(ids_h), dev(probs_h)
    xq = torch.empty((T, H // 32, 40), dtype=torch.uint8, device=DEV)
    gu = torch.empty((T * top_k, 2 * F), dtype=torch.float32, device=DEV)
    hq = torch.empty((T * top_k, F // 32, 40), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, H), dtype=torch.float32, device=DEV)
    ws = qmm.workspace(max(qmm.workspace_bytes(qmm.QMM_OP_MOE_SLOTS, 2 * F, H, T, E, top_k),
                           qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k)), DEV)
    say("graph: routed FFN (quantize, grouped gate||up, swiglu, routed down + combine; fused SwiGLU; moe_ffn)",
        f"E={E} H={H} F={F} T={T} top_k={top_k}")

    ws_f = qmm.workspace(ws.numel(), DEV)
    hq_f = torch.empty_like(hq)
    y_f = torch.empty_like(y)
    ws_l = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MOE_FFN, H, F, T, E, top_k), DEV)
    y_l = torch.empty_like(y)

    def run():
        qmm.q8_1_quantize(x, out=xq)
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, gate_up, xq, ids, out=gu, ws=ws)
        qmm.swiglu_q8_1(gu, out=hq)
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, down, hq, ids, probs, out=y, ws=ws, reuse_routing=True)
        # the same layer with the SwiGLU fused into the gate||up call
        qmm.moe_grouped_swiglu(qmm.QMM_Q4_K, gate_up, xq, ids, out=hq_f, ws=ws_f)
        qmm.moe_grouped_mmq(qmm.QMM_Q4_K, down, hq_f, ids, probs, out=y_f, ws=ws_f, reuse_routing=True)
        # and in one call
        qmm.moe_ffn(qmm.QMM_Q4_K, gate_up, qmm.QMM_Q4_K, down, xq, ids, probs, out=y_l, ws=ws_l)

    # experts relabelled: each token keeps top_k distinct experts
    relabel = torch.randperm(E, generator=torch.Generator().manual_seed(3)).to(torch.int32).to(DEV)

    def change(r):
        x.mul_(0.75 if r % 2 else -1.25)
        if r >= 2:   # new routing: the replay must prepare its route tables again
            ids.copy_(relabel[ids.long()])

    _check_replays(run, [gu, y, hq_f, y_f, y_l], change, "routed FFN")
    assert torch.equal(hq, hq_f) and torch.equal(y, y_f) and torch.equal(y, y_l)
