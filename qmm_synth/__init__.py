"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and places them at the byte offsets of
the block formats. It holds none of the method's arithmetic: no dequantizing,
no activation quantizing, no dot products. Both the CPU oracle and the HIP path
receive exactly the bytes produced here.

Block layouts placed here (little-endian):

* Q4_K super-block, 256 weights in 144 bytes: f16 ``d`` at 0, f16 ``dmin`` at
  2, 12 bytes of packed 6-bit sub-block scales/mins at 4, 128 bytes of 4-bit
  values at 16 (minfer ch. 06 "decode MMVQ: dp4a integer dot products",
  section 3.2, the q4_K kernel's field reads).
* Q5_K super-block, 256 weights in 176 bytes: f16 ``d`` at 0, f16 ``dmin`` at
  2, the 12 packed scale/min bytes at 4, ``qh[32]`` (fifth bits) at 16,
  ``qs[128]`` (4-bit values) at 48 (the pages name the format but not its
  layout; GGUF's is taken).
* Q6_K super-block, 256 weights in 210 bytes: ``ql[128]`` at 0, ``qh[64]`` at
  128, ``sc[16]`` (int8) at 192, f16 ``d`` at 208 (same page, section 3.3,
  the generator-layout pitfall).

Distributions follow the synthetic workloads: ``d``/``dmin`` are |N(0, s)|
rounded to f16, packed scale bytes and 4-bit values are uniform bytes, Q6_K
scales are uniform int8 in [-64, 63], activations are N(0, 1) fp32 with an
optional fraction of outliers multiplied by 20, and the MoE router draws
N(0, 1) logits, takes a float64 softmax and a stable top-k (lower expert index
first on ties).  Draw order is fixed: per weight tensor ``d``, ``dmin``, then
scales, then 4-bit/6-bit payload; then activations; then router logits.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210
Q8_1_BLOCK_BYTES = 40
SUPER_BLOCK = 256
ACT_BLOCK = 32

__all__ = [
    "Q4K_BLOCK_BYTES", "Q5K_BLOCK_BYTES", "Q6K_BLOCK_BYTES", "Q8_1_BLOCK_BYTES", "SUPER_BLOCK", "ACT_BLOCK",
    "rng", "q4k_weights", "q5k_weights", "q6k_weights", "activations", "router", "workload",
    "WORKLOADS",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _abs_normal_f16(g: np.random.Generator, n: int, sigma: float) -> np.ndarray:
    return np.abs(g.normal(0.0, sigma, size=n)).astype(np.float16)


def q4k_weights(g: np.random.Generator, M: int, K: int, d_sigma: float = 0.02) -> np.ndarray:
    """Random Q4_K weight rows: uint8 array of shape [M, K // 256, 144]."""
    if K % SUPER_BLOCK:
        raise ValueError("K must be a multiple of 256")
    nb = M * (K // SUPER_BLOCK)
    d = _abs_normal_f16(g, nb, d_sigma)
    dmin = _abs_normal_f16(g, nb, d_sigma)
    scales = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    out = np.empty((nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = scales
    out[:, 16:144] = qs
    return out.reshape(M, K // SUPER_BLOCK, Q4K_BLOCK_BYTES)


def q5k_weights(g: np.random.Generator, M: int, K: int, d_sigma: float = 0.02) -> np.ndarray:
    """Random Q5_K weight rows: uint8 array of shape [M, K // 256, 176]."""
    if K % SUPER_BLOCK:
        raise ValueError("K must be a multiple of 256")
    nb = M * (K // SUPER_BLOCK)
    d = _abs_normal_f16(g, nb, d_sigma)
    dmin = _abs_normal_f16(g, nb, d_sigma)
    scales = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qh = g.integers(0, 256, size=(nb, 32), dtype=np.uint8)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    out = np.empty((nb, Q5K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = scales
    out[:, 16:48] = qh
    out[:, 48:176] = qs
    return out.reshape(M, K // SUPER_BLOCK, Q5K_BLOCK_BYTES)


def q6k_weights(g: np.random.Generator, M: int, K: int, d_sigma: float = 0.01) -> np.ndarray:
    """Random Q6_K weight rows: uint8 array of shape [M, K // 256, 210]."""
    if K % SUPER_BLOCK:
        raise ValueError("K must be a multiple of 256")
    nb = M * (K // SUPER_BLOCK)
    d = _abs_normal_f16(g, nb, d_sigma)
    sc = g.integers(-64, 64, size=(nb, 16), dtype=np.int8)
    ql = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    qh = g.integers(0, 256, size=(nb, 64), dtype=np.uint8)
    out = np.empty((nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:128] = ql
    out[:, 128:192] = qh
    out[:, 192:208] = sc.view(np.uint8)
    out[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return out.reshape(M, K // SUPER_BLOCK, Q6K_BLOCK_BYTES)


def activations(g: np.random.Generator, T: int, K: int, outlier_frac: float = 0.0,
                outlier_scale: float = 20.0) -> np.ndarray:
    """fp32 activations [T, K] ~ N(0, 1); optional outliers scaled by ``outlier_scale``."""
    x = g.standard_normal(size=(T, K), dtype=np.float32)
    if outlier_frac > 0.0:
        mask = g.random(size=(T, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_scale), x).astype(np.float32)
    return x


def router(g: np.random.Generator, T: int, E: int, top_k: int):
    """Top-k routing from a float64 softmax of N(0, 1) logits.

    Returns ``ids`` int32 [T, top_k] (descending probability, lower expert index
    first on ties) and ``probs`` float32 [T, top_k] (the raw softmax
    probabilities of the chosen experts, not renormalised).
    """
    logits = g.standard_normal(size=(T, E))
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    ids = order.astype(np.int32)
    probs = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, probs


# The five synthetic workloads. Sizes and distributions as stated in the
# module docstring; ``seed`` is the workload's index.
WORKLOADS = {
    0: dict(name="q4k_gemv_1024", kind="mmvq", fmt="q4k", M=1024, K=1024, T=(1,)),
    1: dict(name="decode_mmvq_4096x11008", kind="mmvq", fmt=("q4k", "q6k"), M=4096, K=11008, T=(1, 4)),
    2: dict(name="prefill_mmq_4096x4096_t512", kind="mmq", fmt="q4k", M=4096, K=4096, T=512),
    3: dict(name="prefill_mmq_ffn_up_t1024", kind="mmq", fmt=("q4k", "q6k"),
            shapes={"q4k": (14336, 4096), "q6k": (4096, 14336)}, T=1024, outlier_frac=0.01),
    4: dict(name="moe_grouped_e128_t512_top8", kind="moe", fmt="q4k", E=128, hidden=2048,
            ffn=768, T=512, top_k=8),
}


def workload(idx: int, T: int | None = None, rows: int | None = None, experts: int | None = None) -> dict:
    """Materialise workload ``idx`` with seed ``idx``.

    ``rows`` truncates the weight row count (MMVQ/MMQ) and ``experts`` the
    expert count (MoE) for bounded samples; ``T`` overrides the token count.
    Truncation draws the same kind of data, not a prefix of the full draw.
    """
    w = WORKLOADS[idx]
    g = rng(idx)
    out: dict = {"spec": w}
    if idx == 0:
        M = rows or w["M"]
        out["q4k"] = q4k_weights(g, M, w["K"])
        out["x"] = activations(g, T or 1, w["K"])
    elif idx == 1:
        M = rows or w["M"]
        out["q4k"] = q4k_weights(g, M, w["K"])
        out["q6k"] = q6k_weights(g, M, w["K"])
        out["x"] = activations(g, T or max(w["T"]), w["K"])
        out["q5k"] = q5k_weights(g, M, w["K"])      # drawn last: the tensors above keep their bytes
    elif idx == 2:
        M = rows or w["M"]
        out["q4k"] = q4k_weights(g, M, w["K"])
        out["x"] = activations(g, T or w["T"], w["K"])
    elif idx == 3:
        (M4, K4), (M6, K6) = w["shapes"]["q4k"], w["shapes"]["q6k"]
        out["q4k"] = q4k_weights(g, rows or M4, K4)
        out["q6k"] = q6k_weights(g, rows or M6, K6)
        t = T or w["T"]
        out["x_q4k"] = activations(g, t, K4, outlier_frac=w["outlier_frac"])
        out["x_q6k"] = activations(g, t, K6, outlier_frac=w["outlier_frac"])
    elif idx == 4:
        E = experts or w["E"]
        H, F = w["hidden"], w["ffn"]
        # gate and up are drawn as one [2F, H] tensor per expert (rows 0..F-1
        # gate, F..2F-1 up); down is [H, F] per expert.
        out["gate_up"] = np.stack([q4k_weights(g, 2 * F, H) for _ in range(E)])
        out["down"] = np.stack([q4k_weights(g, H, F) for _ in range(E)])
        t = T or w["T"]
        out["x"] = activations(g, t, H)
        ids, probs = router(g, t, E, w["top_k"])
        out["ids"], out["probs"] = ids, probs
    return out
