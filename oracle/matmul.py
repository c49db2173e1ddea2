"""Dense results, error bounds and integer sub-block sums (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method's result has a plain definition: with ``W`` the dequantised
weights [M, K] and ``X`` the dequantised Q8_1 activations [T, K],

    y[t, i] = sum_k W[i, k] * X[t, k]          (fp64 here)

stored as ``y[t * M + i]`` ([8e] §3.2: one output row per weight row, token
major).  The kernels reach it through the factorisation of [8e] §2 (the
min-term paragraph): per 32-weight sub-block ``s`` of a Q4_K row,

    W.x = sum_s [ d*sc_s*dx_s*D_s - dmin*m_s*dx_s*S_s ],
    D_s = sum_{e in s} nib_e * q_e,  S_s = sum_{e in s} q_e,

so the integer sums ``D`` and ``S`` are unique and checked bit for bit, and
the floating result is checked against ``dense`` within
``1e-4 * abs_bound`` per element.
"""
from __future__ import annotations

import numpy as np

from .formats import q4k_fields, q5k_fields, q6k_fields, q8_1_fields


def dense(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """``y[t, i] = sum_k W[i, k] X[t, k]`` in float64; returns [T, M]."""
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64).T


def abs_bound(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """``sum_k |W[i, k]| |X[t, k]|`` in float64; the per-element error scale."""
    return np.abs(np.asarray(X, np.float64)) @ np.abs(np.asarray(W, np.float64)).T


def q4k_subdots(wblocks: np.ndarray, xq: np.ndarray):
    """Integer sub-block sums of a Q4_K x Q8_1 product.

    ``wblocks[M, K/256, 144]``, ``xq[T, K/32, 40]``.  Returns
    ``D[T, M, K/32] = sum_{e in s} nib[i, e] q[t, e]`` and
    ``S[T, K/32] = sum_{e in s} q[t, e]`` (int64, exact).
    """
    M, nb = wblocks.shape[0], wblocks.shape[1]
    _, _, _, _, nib = q4k_fields(wblocks)
    nib = nib.reshape(M, nb * 8, 32)
    _, q, _, _ = q8_1_fields(xq)          # [T, K/32, 32]
    D = np.einsum("isk,tsk->tis", nib, q, dtype=np.int64)
    S = q.sum(axis=-1)
    return D, S


def q6k_subdots(wblocks: np.ndarray, xq: np.ndarray):
    """Integer 16-weight sub-block sums ``D6[T, M, K/16] = sum (q6 - 32) q`` (int64)."""
    M, nb = wblocks.shape[0], wblocks.shape[1]
    _, _, q6 = q6k_fields(wblocks)
    w = (q6 - 32).reshape(M, nb * 16, 16)
    _, q, _, _ = q8_1_fields(xq)
    T = q.shape[0]
    q16 = q.reshape(T, -1, 16)
    return np.einsum("isk,tsk->tis", w, q16, dtype=np.int64)


def q4k_factored(wblocks: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """``y`` rebuilt from the integer sums through the min-term factorisation (fp64)."""
    M, nb = wblocks.shape[0], wblocks.shape[1]
    d, dmin, sc, m, _ = q4k_fields(wblocks)           # d,dmin [M, nb]; sc,m [M, nb, 8]
    D, S = q4k_subdots(wblocks, xq)                   # [T, M, nb*8], [T, nb*8]
    dx, _, _, _ = q8_1_fields(xq)                     # [T, nb*8]
    scale = (d[:, :, None] * sc).reshape(M, nb * 8)   # d * sc_s
    mins = (dmin[:, :, None] * m).reshape(M, nb * 8)  # dmin * m_s
    main = (dx[:, None, :] * scale[None] * D).sum(axis=-1)
    corr = (dx * S) @ mins.T
    return main - corr


def q6k_factored(wblocks: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """``y = sum_{s16} d * sc_{s16} * dx_{s16 // 2} * D6_{s16}`` (fp64)."""
    M, nb = wblocks.shape[0], wblocks.shape[1]
    d, sc, _ = q6k_fields(wblocks)                    # d [M, nb], sc [M, nb, 16]
    D6 = q6k_subdots(wblocks, xq)                     # [T, M, nb*16]
    dx, _, _, _ = q8_1_fields(xq)                     # [T, nb*8]
    dx16 = np.repeat(dx, 2, axis=-1)                  # 32-block scale for each 16-sub-block
    scale = (d[:, :, None] * sc).reshape(M, nb * 16)
    return (dx16[:, None, :] * scale[None] * D6).sum(axis=-1)


def q5k_subdots(wblocks: np.ndarray, xq: np.ndarray):
    """Integer sub-block sums of a Q5_K x Q8_1 product: ``D[T, M, K/32] = sum q5 q``, ``S[T, K/32]``."""
    M, nb = wblocks.shape[0], wblocks.shape[1]
    _, _, _, _, q5 = q5k_fields(wblocks)
    q5 = q5.reshape(M, nb * 8, 32)
    _, q, _, _ = q8_1_fields(xq)
    D = np.einsum("isk,tsk->tis", q5, q, dtype=np.int64)
    S = q.sum(axis=-1)
    return D, S


def q5k_factored(wblocks: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """``y`` from the Q5_K integer sums through the min-term factorisation of [8e] §2 (fp64)."""
    M, nb = wblocks.shape[0], wblocks.shape[1]
    d, dmin, sc, m, _ = q5k_fields(wblocks)
    D, S = q5k_subdots(wblocks, xq)
    dx, _, _, _ = q8_1_fields(xq)
    scale = (d[:, :, None] * sc).reshape(M, nb * 8)
    mins = (dmin[:, :, None] * m).reshape(M, nb * 8)
    main = (dx[:, None, :] * scale[None] * D).sum(axis=-1)
    corr = (dx * S) @ mins.T
    return main - corr
