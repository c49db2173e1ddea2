"""MoE routed-expert grouping, grouped products and the weighted combine (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GAP] "T2 -- Tensor-core grouped MoE expert GEMM" and its de-risk paragraph
describe the grouped path: count the tokens routed to each expert, turn the
counts into offsets with a prefix sum, list the token slots per expert, run
one product per expert so each expert's weights are read once, and scatter
the results back.  [MMQ] "MoE routing (fused gather)" gathers the activations
by expert.  The oracle states each step plainly:

* slot ``s = t * top_k + k`` is token ``t``'s ``k``-th routed expert
  ``ids[t, k]``;
* ``route_buckets`` lists slots per expert in increasing slot order;
* ``grouped`` gives ``y_slot[s] = W[ids[t, k]] . x_row`` where the activation
  row is ``t`` (one row per token, gate/up) or ``s`` (one row per slot, down);
* ``combine`` gives ``y[t] = sum_k p[t, k] * y_slot[t * top_k + k]`` summed
  in increasing ``k``.
"""
from __future__ import annotations

import numpy as np


def route_buckets(ids: np.ndarray, E: int):
    """Histogram, exclusive prefix sum and per-expert slot lists.

    Returns ``counts[E]``, ``offsets[E + 1]`` and ``bucket[T * top_k]`` with
    the slots of expert ``e`` at ``bucket[offsets[e]:offsets[e + 1]]`` in
    increasing order.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    bucket = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for s, e in enumerate(flat):          # plain loop: slots in increasing order
        bucket[fill[e]] = s
        fill[e] += 1
    return counts, offsets, bucket


def grouped(W: np.ndarray, X: np.ndarray, ids: np.ndarray, rows_per_token: int) -> np.ndarray:
    """Per-slot products ``y_slot[T * top_k, M]`` (fp64).

    ``W[E, M, K]`` dequantised expert weights, ``X[R, K]`` dequantised
    activations with ``R = T`` (``rows_per_token == 1``) or ``R = T * top_k``.
    """
    T, top_k = ids.shape
    E, M, _ = W.shape
    out = np.zeros((T * top_k, M), dtype=np.float64)
    _, offsets, bucket = route_buckets(ids, E)
    for e in range(E):
        slots = bucket[offsets[e]:offsets[e + 1]]
        if slots.size == 0:
            continue
        rows = slots // top_k if rows_per_token == 1 else slots
        out[slots] = np.asarray(X, np.float64)[rows] @ np.asarray(W[e], np.float64).T
    return out


def combine(y_slot: np.ndarray, probs: np.ndarray) -> np.ndarray:
    """``y[t] = sum_k p[t, k] * y_slot[t * top_k + k]`` with k ascending (fp64)."""
    T, top_k = probs.shape
    ys = np.asarray(y_slot, np.float64).reshape(T, top_k, -1)
    p = np.asarray(probs, np.float64)
    y = np.zeros((T, ys.shape[-1]), dtype=np.float64)
    for k in range(top_k):
        y = y + p[:, k:k + 1] * ys[:, k, :]
    return y


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``silu(gate) * up = gate / (1 + exp(-gate)) * up`` in float64 (glue reading)."""
    g = np.asarray(gate, np.float64)
    with np.errstate(over="ignore"):      # exp(-g) -> inf gives the exact limit -0
        return g / (1.0 + np.exp(-g)) * np.asarray(up, np.float64)


def grouped_blocks(dequant, blocks: np.ndarray, X: np.ndarray, ids: np.ndarray,
                   rows_per_token: int, experts=None):
    """``grouped`` for quantized expert weights, one expert dequantised at a time.

    ``dequant`` maps one expert's blocks to float64 [M, K] (``q4k_dequant`` or
    ``q6k_dequant``).  Returns ``(y_slot, bound)`` with
    ``bound[s] = sum_k |W[e]| |x_row|`` (the per-element error scale); only
    the slots of ``experts`` (all by default) are filled.
    """
    T, top_k = ids.shape
    E = blocks.shape[0]
    M = blocks.shape[1]
    y = np.zeros((T * top_k, M), dtype=np.float64)
    bound = np.zeros((T * top_k, M), dtype=np.float64)
    _, offsets, bucket = route_buckets(ids, E)
    Xf = np.asarray(X, np.float64)
    for e in (range(E) if experts is None else experts):
        slots = bucket[offsets[e]:offsets[e + 1]]
        if slots.size == 0:
            continue
        W = dequant(blocks[e])
        rows = slots // top_k if rows_per_token == 1 else slots
        y[slots] = Xf[rows] @ W.T
        bound[slots] = np.abs(Xf[rows]) @ np.abs(W).T
    return y, bound
