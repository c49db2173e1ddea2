#!/usr/bin/env python3
"""Benchmark of the fused-dequant Q4_K / Q6_K x Q8_1 hot path on one MI355X.

Headline workload (the decode matvec shape the metric is quoted on):
W 4096 x 11008 in Q4_K and the same shape in Q6_K, x fp32 N(0, 1) of length
11008, T = 1.  One step = quantize x to Q8_1, then the Q4_K and the Q6_K
matvec (the whole decode path), with inputs resident in HBM.  The weights
rotate over enough copies (> 512 MB) that no step reads them from the
256 MB Infinity Cache.  Steps are captured in one HIP graph and replayed;
HIP events bracket the replay.  `value` is algorithmic bytes per step
(quantized weights + Q8_1 activations + fp32 input/outputs) over step time.

The same JSON line carries:
  roofline      the dominant kernel (the Q6_K matvec, 37 MB per launch):
                algorithmic bytes over its launch duration (HIP events
                around a graph of back-to-back launches on the launch
                stream, divided by the launch count), against 8 TB/s HBM;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same
                decode workload (whole passes over both matrices, repeated
                for about 10 s), in GB/s;
  also          the other kernels and workloads measured the same way:
                matvec at T = 4, the Q5_K matvec (T = 1, 4) and GEMM
                (4096 x 4096, T = 512), matvec vs GEMM at T = 8 (the small-T
                crossover), the read-only HBM ceiling probe at the
                matvec byte counts, the prefill GEMMs (int8 TOPS and
                tokens/s at T = 512 / 1024; also from fp32 activations:
                quantize + GEMM vs the fused quantizer), the routed-expert
                MoE FFN, and the per-slot expert matvec vs grouped GEMM
                comparator at expert shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MMVQ HBM GB/s (T=1) + MMQ int8 TOPS & tokens/s at T=512/1024, %roofline"
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
MALL_BYTES = 256 << 20
# Weight copies rotated per launch.  The Infinity Cache (MALL, 256 MB) does
# not evict strictly LRU: a cyclic working set of 2x its size still hits
# measurably (apparent bandwidth above the HBM peak), so the rotation spans
# 16x the MALL.
ROTATE_BYTES = 4096 << 20

# traffic measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE for the
# dominant kernel (profiles/); None until taken for the current kernel
DOMINANT_TRAFFIC_BYTES = 37436825   # mmvq_q6k, profiles/mmvq_decode_4096x11008_t1.md


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_graph(torch, fns, reps, warm=2):
    """Capture fns[i % len(fns)] for i < reps into one graph; return ms per call."""
    for i in range(warm):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    a, b = _events(torch)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_launches(torch, fns, reps, sleep_cycles):
    """Mean and median ms of single launches bracketed by event pairs.

    A spin kernel first keeps the GPU busy while all (event, launch, event)
    triples are enqueued, so each pair brackets its kernel with no host gap.
    """
    evs = [_events(torch) for _ in range(reps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    for i in range(reps):
        evs[i][0].record()
        fns[i % len(fns)]()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(ms) / len(ms), ms[len(ms) // 2]


def calibrate_sleep(torch):
    a, b = _events(torch)
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(1_000_000)
    b.record()
    torch.cuda.synchronize()
    return max(1e-4, a.elapsed_time(b)) / 1_000_000   # ms per cycle


def copies_for(nbytes):
    return max(2, math.ceil(ROTATE_BYTES / max(1, nbytes)) + 1)


def rotated(t, n):
    """n device copies of tensor t (made on the device)."""
    return [t] + [t.clone() for _ in range(n - 1)]


def cpu_oracle_baseline(np, wl, rows, min_seconds=10.0, one_core=False):
    """The fp64 oracle on the first `rows` rows of both decode matrices, T = 1
    (on all BLAS threads, or with the BLAS limited to one thread)."""
    if one_core:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            r = cpu_oracle_baseline(np, wl, rows, min_seconds)
        r["cores"] = 1
        r["sample"] = r["sample"].replace("matvec on the BLAS threads", "matvec on one BLAS thread")
        return r
    import oracle
    try:
        import threadpoolctl
        a = np.ones((64, 64))
        _ = a @ a
        cores = max([i["num_threads"] for i in threadpoolctl.threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    x = wl["x"][:1]
    reps, t0 = 0, time.perf_counter()
    while True:
        xq = oracle.quantize_q8_1(x)
        X = oracle.q8_1_dequant(xq)
        y4 = oracle.dense(oracle.q4k_dequant(wl["q4k"][:rows]), X)
        y6 = oracle.dense(oracle.q6k_dequant(wl["q6k"][:rows]), X)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 50:
            break
    del y4, y6
    K = x.shape[1]
    nbytes = reps * (rows * (K // 256) * (144 + 210) + 2 * (xq.nbytes + rows * 4) + x.nbytes)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{reps} passes over rows 0..{rows - 1} of the 4096x11008 Q4_K and Q6_K "
                      f"matrices at T=1 (quantize, fp64 dequantize, fp64 matvec), {dt:.1f} s wall; "
                      "dequantization single-threaded numpy, matvec on the BLAS threads"}


def moe_comparator(torch, qmm, qmm_synth, dev):
    """Per-slot expert matvec vs grouped GEMM at expert shapes.

    128 experts of M x 2048 Q4_K (M = 512, 704), top-8, balanced routing with
    exactly N tokens per expert (N = 8..64, T = 16 N tokens): slot t*8 + k goes
    to expert (t*8 + k) mod 128.  Both calls produce the per-slot rows; the
    grouped call includes its route preparation and activation repack.
    Weights rotate over >= 4 GB of copies.
    """
    import numpy as np
    E, K, top_k = 128, 2048, 8
    out = {}
    for M in (512, 704):
        g = qmm_synth.rng(40 + M)
        w1 = np.stack([qmm_synth.q4k_weights(g, M, K) for _ in range(E)])
        wd = torch.from_numpy(w1).to(dev)
        R = copies_for(w1.nbytes)
        ws_ = rotated(wd, R)
        for N in (8, 16, 32, 64):
            T = E * N // top_k
            ids = torch.from_numpy((np.arange(T * top_k, dtype=np.int32) % E).reshape(T, top_k)).to(dev)
            xq = qmm.q8_1_quantize(torch.from_numpy(qmm_synth.activations(g, T, K)).to(dev))
            y = torch.empty((T * top_k, M), dtype=torch.float32, device=dev)
            wsp = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MOE, M, K, T, E, top_k), dev)
            t_mv = time_graph(torch, [lambda c=c: qmm.moe_slot_mmvq(qmm.QMM_Q4_K, ws_[c], xq, ids, out=y)
                                      for c in range(R)], 100)
            t_gr = time_graph(torch, [lambda c=c: qmm.moe_grouped_mmq(qmm.QMM_Q4_K, ws_[c], xq, ids, out=y, ws=wsp)
                                      for c in range(R)], 100)
            out[f"M{M}_N{N}"] = {"slot_matvec_us": round(t_mv * 1e3, 2), "grouped_us": round(t_gr * 1e3, 2),
                                 "grouped_speedup": round(t_mv / t_gr, 2)}
            log(f"moe comparator M={M} N={N}: slot matvec {t_mv * 1e3:.1f} us, grouped {t_gr * 1e3:.1f} us")
        del ws_, wd
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the secondary workloads (for profiling the decode step)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="after the headline, only the prefill GEMMs and the routed-expert FFN (for counter runs)")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU sharding is a design "
                                   "note only (row split for matvec/GEMM, expert split for MoE)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import qmm_synth
    import quantized_matmul_q8_amd as qmm

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    cyc_ms = calibrate_sleep(torch)
    log(f"sleep calibration: {cyc_ms * 1e6:.3f} ns per cycle")

    # ---------------- headline: decode step at T = 1 ----------------
    wl = qmm_synth.workload(1)
    M, K = 4096, 11008
    w4h, w6h = wl["q4k"], wl["q6k"]
    step_w_bytes = w4h.nbytes + w6h.nbytes
    R = copies_for(step_w_bytes)
    w4 = rotated(to(w4h), R)
    w6 = rotated(to(w6h), R)
    x1 = to(wl["x"][:1])
    xq1 = torch.empty((1, K // 32, 40), dtype=torch.uint8, device=dev)
    y4 = torch.empty((1, M), dtype=torch.float32, device=dev)
    y6 = torch.empty((1, M), dtype=torch.float32, device=dev)

    def make_step(c):
        def step():
            qmm.q8_1_quantize(x1, out=xq1)
            qmm.mmvq_q4k(w4[c], xq1, out=y4)
            qmm.mmvq_q6k(w6[c], xq1, out=y6)
        return step

    steps = [make_step(c) for c in range(R)]
    for i in range(args.warmup):
        steps[i % R]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(args.steps):
            steps[i % R]()
    g.replay()                      # graph warm-up (untimed)
    torch.cuda.synchronize()
    a, b = _events(torch)
    torch.cuda.synchronize()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / args.steps
    log(f"decode step: {ms_step * 1e3:.3f} us per step over {args.steps} graph-replayed steps")
    xq_bytes = (K // 32) * 40
    bytes_q4 = w4h.nbytes + xq_bytes + M * 4
    bytes_q6 = w6h.nbytes + xq_bytes + M * 4
    bytes_quant = K * 4 + xq_bytes
    step_bytes = bytes_q4 + bytes_q6 + bytes_quant
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: Q6_K matvec, per-launch event pairs on the launch stream
    n_launch = 120
    sleep = int(max(4.0, n_launch * 0.1) / cyc_ms)
    q6_fns = [lambda c=c: qmm.mmvq_q6k(w6[c], xq1, out=y6) for c in range(R)]
    q4_fns = [lambda c=c: qmm.mmvq_q4k(w4[c], xq1, out=y4) for c in range(R)]
    # launch duration = HIP events around a graph of back-to-back launches
    # (rotating weight copies) / launches; this agrees with rocprofv3's
    # kernel durations.  Per-launch event pairs add the dispatch overhead
    # of the event packets and are reported beside it.
    q6_graph = time_graph(torch, q6_fns, 200)
    q4_graph = time_graph(torch, q4_fns, 200)
    q6_mean, q6_med = time_launches(torch, q6_fns, n_launch, sleep)
    ach = bytes_q6 / (q6_graph * 1e-3) / 1e9
    roofline = {"kernel": "mmvq_q6k (4096x11008, T=1)", "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": DOMINANT_TRAFFIC_BYTES, "algorithmic_bytes": bytes_q6,
                "launch_us": round(q6_graph * 1e3, 3),
                "event_pair_mean_us": round(q6_mean * 1e3, 3)}

    log(f"mmvq_q6k {q6_graph * 1e3:.3f} us (graph), {q6_mean * 1e3:.3f} us (event pairs); "
        f"mmvq_q4k {q4_graph * 1e3:.3f} us")
    also = {}

    def gbps(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    also["mmvq_q4k_t1"] = {"us": round(q4_graph * 1e3, 3), "GBps": gbps(bytes_q4, q4_graph),
                           "frac_hbm": round(gbps(bytes_q4, q4_graph) / HBM_PEAK_GBPS, 4)}
    also["mmvq_q6k_t1"] = {"us": round(q6_graph * 1e3, 3), "GBps": round(ach, 1),
                           "frac_hbm": round(ach / HBM_PEAK_GBPS, 4)}

    # read-only ceiling at the same byte counts (rotating buffers)
    for name, nb in (("probe_read_25MB", w4h.nbytes), ("probe_read_37MB", w6h.nbytes)):
        nb16 = nb // 16 * 16
        bufs = rotated(torch.zeros((nb16,), dtype=torch.uint8, device=dev), copies_for(nb16))
        sink = torch.zeros((4,), dtype=torch.int32, device=dev)
        fns = [lambda b_=b_: qmm.probe_read(b_, nb16, sink) for b_ in bufs]
        pm = time_graph(torch, fns, 200)
        also[name] = {"us": round(pm * 1e3, 3), "GBps": gbps(nb16, pm),
                      "frac_hbm": round(gbps(nb16, pm) / HBM_PEAK_GBPS, 4)}
        del bufs

    if not args.only_headline and not args.prefill_only:
        # single Q4_K matvec 1024 x 1024, T = 1 (reported only: launch-latency bound)
        wl0 = qmm_synth.workload(0)
        w0h = wl0["q4k"]
        # one launch per copy, every copy distinct (about 7,000 copies, 4 GB, so
        # no launch finds its weights in the MALL)
        n0 = copies_for(w0h.nbytes)
        w0 = to(w0h).unsqueeze(0).repeat(n0, 1, 1, 1)
        xq0 = qmm.q8_1_quantize(to(wl0["x"]))
        y0 = torch.empty((1, w0h.shape[0]), dtype=torch.float32, device=dev)
        m_ = time_graph(torch, [lambda c=c: qmm.mmvq_q4k(w0[c], xq0, out=y0) for c in range(n0)], n0)
        nbytes = w0h.nbytes + xq0.numel() + y0.numel() * 4
        also["mmvq_q4k_1024x1024_t1"] = {"us": round(m_ * 1e3, 3), "GBps": gbps(nbytes, m_),
                                         "frac_hbm": round(gbps(nbytes, m_) / HBM_PEAK_GBPS, 4)}
        del w0, wl0

    if not args.only_headline and not args.prefill_only:
        # matvec at T = 4
        x4 = to(wl["x"][:4])
        xq4 = qmm.q8_1_quantize(x4)
        y44 = torch.empty((4, M), dtype=torch.float32, device=dev)
        for name, ws_, fn, nbw in (("mmvq_q4k_t4", w4, qmm.mmvq_q4k, w4h.nbytes),
                                    ("mmvq_q6k_t4", w6, qmm.mmvq_q6k, w6h.nbytes)):
            fns = [lambda c=c, ws_=ws_, fn=fn: fn(ws_[c], xq4, out=y44) for c in range(R)]
            m_ = time_graph(torch, fns, 200)
            nbytes = nbw + 4 * xq_bytes + 4 * M * 4
            also[name] = {"us": round(m_ * 1e3, 3), "GBps": gbps(nbytes, m_),
                          "frac_hbm": round(gbps(nbytes, m_) / HBM_PEAK_GBPS, 4)}

        # third format: Q5_K matvec on the decode shape, T = 1 and 4
        w5h = wl["q5k"]
        w5 = rotated(to(w5h), copies_for(w5h.nbytes))
        for name, xq_, T_ in (("mmvq_q5k_t1", xq1, 1), ("mmvq_q5k_t4", xq4, 4)):
            y5 = torch.empty((T_, M), dtype=torch.float32, device=dev)
            m_ = time_graph(torch, [lambda c=c, xq_=xq_, y5=y5: qmm.mmvq_q5k(w5[c], xq_, out=y5)
                                    for c in range(len(w5))], 200)
            nbytes = w5h.nbytes + T_ * xq_bytes + T_ * M * 4
            also[name] = {"us": round(m_ * 1e3, 3), "GBps": gbps(nbytes, m_),
                          "frac_hbm": round(gbps(nbytes, m_) / HBM_PEAK_GBPS, 4)}
        del w5

        # small-T crossover on the decode shape: matvec vs GEMM at T = 8
        x8 = to(qmm_synth.activations(qmm_synth.rng(8), 8, K))
        xq8 = qmm.q8_1_quantize(x8)
        y8 = torch.empty((8, M), dtype=torch.float32, device=dev)
        ws8 = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MMQ, M, K, 8), dev)
        cross = {}
        for key, ws_, mv, mq, nbw in (("q4k", w4, qmm.mmvq_q4k, qmm.mmq_q4k, w4h.nbytes),
                                      ("q6k", w6, qmm.mmvq_q6k, qmm.mmq_q6k, w6h.nbytes)):
            t_mv = time_graph(torch, [lambda c=c: mv(ws_[c], xq8, out=y8) for c in range(R)], 200)
            t_mq = time_graph(torch, [lambda c=c: mq(ws_[c], xq8, out=y8, ws=ws8) for c in range(R)], 200)
            cross[f"mmvq_{key}_us"] = round(t_mv * 1e3, 2)
            cross[f"mmq_{key}_us"] = round(t_mq * 1e3, 2)
            cross[f"best_{key}_GBps"] = gbps(nbw, min(t_mv, t_mq))
        also["decode_4096x11008_t8"] = cross
    del w4, w6

    if not args.only_headline:
        # prefill GEMMs
        def mmq_case(name, fn, wh, xh):
            Mg, Kg = wh.shape[0], wh.shape[1] * 256
            Tg = xh.shape[0]
            cop = 4
            wd = [to(wh) for _ in range(cop)]
            xqg = qmm.q8_1_quantize(to(xh))
            yg = torch.empty((Tg, Mg), dtype=torch.float32, device=dev)
            fns = [lambda c=c: fn(wd[c], xqg, out=yg) for c in range(cop)]
            mean = time_graph(torch, fns, 20)
            ops = 2.0 * Mg * Kg * Tg
            tops = ops / (mean * 1e-3) / 1e12
            log(f"{name}: {mean * 1e3:.2f} us")
            also[name] = {"us": round(mean * 1e3, 2),
                          "TOPS": round(tops, 1), "frac_int8": round(tops / INT8_PEAK_TOPS, 4),
                          "tokens_per_s": round(Tg / (mean * 1e-3), 1)}
            del wd

        wl2 = qmm_synth.workload(2)
        mmq_case("mmq_q4k_4096x4096_t512", qmm.mmq_q4k, wl2["q4k"], wl2["x"])
        mmq_case("mmq_q5k_4096x4096_t512", qmm.mmq_q5k, qmm_synth.q5k_weights(qmm_synth.rng(52), 4096, 4096),
                 wl2["x"])
        # fused quantizer prologue: fp32 activations in, against quantize + GEMM
        wd2 = [to(wl2["q4k"]) for _ in range(4)]
        x2 = to(wl2["x"])
        xq2 = torch.empty((x2.shape[0], x2.shape[1] // 32, 40), dtype=torch.uint8, device=dev)
        y2g = torch.empty((x2.shape[0], wl2["q4k"].shape[0]), dtype=torch.float32, device=dev)

        def two_pass(c):
            qmm.q8_1_quantize(x2, out=xq2)
            qmm.mmq_q4k(wd2[c], xq2, out=y2g)

        t_two = time_graph(torch, [lambda c=c: two_pass(c) for c in range(4)], 20)
        t_fused = time_graph(torch, [lambda c=c: qmm.mmq_q4k_f32(wd2[c], x2, out=y2g) for c in range(4)], 20)
        also["mmq_q4k_4096x4096_t512_from_fp32"] = {"quantize_then_gemm_us": round(t_two * 1e3, 2),
                                                     "fused_us": round(t_fused * 1e3, 2)}
        del wd2
        del wl2
        wl3 = qmm_synth.workload(3)
        mmq_case("mmq_q4k_14336x4096_t1024", qmm.mmq_q4k, wl3["q4k"], wl3["x_q4k"])
        mmq_case("mmq_q6k_4096x14336_t1024", qmm.mmq_q6k, wl3["q6k"], wl3["x_q6k"])
        del wl3

        # routed-expert FFN: gate||up grouped, SwiGLU->Q8_1, down grouped weighted
        wl4 = qmm_synth.workload(4)
        E, H, F, T, top_k = 128, 2048, 768, 512, 8
        gu = to(wl4["gate_up"])
        dn = to(wl4["down"])
        ids = to(wl4["ids"])
        probs = to(wl4["probs"])
        xm = to(wl4["x"])
        xqm = torch.empty((T, H // 32, 40), dtype=torch.uint8, device=dev)
        y1 = torch.empty((T * top_k, 2 * F), dtype=torch.float32, device=dev)
        hq = torch.empty((T * top_k, F // 32, 40), dtype=torch.uint8, device=dev)
        y2 = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws1 = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MOE, 2 * F, H, T, E, top_k), dev)
        ws2 = qmm.workspace(qmm.workspace_bytes(qmm.QMM_OP_MOE, H, F, T, E, top_k), dev)

        def moe_step():
            qmm.q8_1_quantize(xm, out=xqm)
            qmm.moe_grouped_mmq(qmm.QMM_Q4_K, gu, xqm, ids, out=y1, ws=ws1)
            qmm.swiglu_q8_1(y1, out=hq)
            qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dn, hq, ids, probs, out=y2, ws=ws2)

        def gate_up_only():
            qmm.moe_grouped_mmq(qmm.QMM_Q4_K, gu, xqm, ids, out=y1, ws=ws1)

        def down_only():
            qmm.moe_grouped_mmq(qmm.QMM_Q4_K, dn, hq, ids, probs, out=y2, ws=ws2)

        def glue_only():
            qmm.q8_1_quantize(xm, out=xqm)
            qmm.swiglu_q8_1(y1, out=hq)

        log("moe ffn")
        ms_moe = time_graph(torch, [moe_step], 10)
        ms_gu = time_graph(torch, [gate_up_only], 10)
        ms_dn = time_graph(torch, [down_only], 10)
        ms_glue = time_graph(torch, [glue_only], 10)
        wbytes = wl4["gate_up"].nbytes + wl4["down"].nbytes
        macs = T * top_k * (2 * F * H + H * F)
        act_bytes = T * H * 4 + T * (H // 32) * 40 + T * top_k * (F // 32) * 40 + T * H * 4
        moe_bytes = wbytes + act_bytes
        tops = 2.0 * macs / (ms_moe * 1e-3) / 1e12
        attain = min(INT8_PEAK_TOPS, 2.0 * macs / moe_bytes * HBM_PEAK_GBPS / 1e3)
        # the two grouped calls alone (route preparation, repack, GEMM and, for
        # down, the combine), without the quantize and SwiGLU glue: weights,
        # Q8_1 inputs, the gate||up per-slot rows and the combined output
        g_bytes = wbytes + T * (H // 32) * 40 + T * top_k * 2 * F * 4 + T * top_k * (F // 32) * 40 + T * H * 4
        ms_g = ms_gu + ms_dn
        tops_g = 2.0 * macs / (ms_g * 1e-3) / 1e12
        attain_g = min(INT8_PEAK_TOPS, 2.0 * macs / g_bytes * HBM_PEAK_GBPS / 1e3)
        also["moe_ffn_e128_t512_top8"] = {
            "us": round(ms_moe * 1e3, 2), "gate_up_us": round(ms_gu * 1e3, 2),
            "down_us": round(ms_dn * 1e3, 2), "GBps": gbps(moe_bytes, ms_moe),
            "frac_hbm": round(gbps(moe_bytes, ms_moe) / HBM_PEAK_GBPS, 4),
            "TOPS": round(tops, 1), "frac_attainable": round(tops / attain, 4),
            "tokens_per_s": round(T / (ms_moe * 1e-3), 1),
            "glue_us": round(ms_glue * 1e3, 2),
            "grouped_calls_only": {"us": round(ms_g * 1e3, 2), "GBps": gbps(g_bytes, ms_g),
                                   "TOPS": round(tops_g, 1), "frac_attainable": round(tops_g / attain_g, 4)}}
        del gu, dn
        if not args.prefill_only:
            also["moe_comparator_e128_k2048_top8"] = moe_comparator(torch, qmm, qmm_synth, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu oracle baseline")
        cpu = cpu_oracle_baseline(np, wl, min(args.cpu_rows, M))
        also["cpu_oracle_1core"] = cpu_oracle_baseline(np, wl, min(args.cpu_rows, M), min_seconds=5.0, one_core=True)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "decode_mmvq_4096x11008_q4k+q6k_t1", "M": M, "K": K, "T": 1,
                   "step": "q8_1_quantize + mmvq_q4k + mmvq_q6k", "step_bytes": step_bytes,
                   "weight_copies_rotated": R, "parallelism": "single_gpu"},
        "roofline": roofline, "cpu_baseline": cpu, "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
