"""Decoders for the Q4_K, Q5_K, Q6_K and Q8_1 block formats (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

All decoders take uint8 arrays whose last axis is one block and return the
block's fields as int64 / float64 arrays.  Nothing is vectorised beyond numpy
indexing, so each line can be checked against the layout it states.
"""
from __future__ import annotations

import numpy as np

Q4K_BYTES = 144
Q5K_BYTES = 176
Q6K_BYTES = 210
Q8_1_BYTES = 40


def _f16_at(b: np.ndarray, off: int) -> np.ndarray:
    """Little-endian IEEE binary16 at byte offset ``off`` of the last axis, as float64."""
    two = np.ascontiguousarray(b[..., off:off + 2])
    return two.view("<f2")[..., 0].astype(np.float64)


def _scales_mins(packed: np.ndarray):
    """Eight 6-bit scales and mins from the 12 packed bytes of a Q4_K / Q5_K block."""
    S = packed.astype(np.int64)
    sc = np.empty(S.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty(S.shape[:-1] + (8,), dtype=np.int64)
    sc[..., 0:4] = S[..., 0:4] & 63
    m[..., 0:4] = S[..., 4:8] & 63
    sc[..., 4:8] = (S[..., 8:12] & 15) | ((S[..., 0:4] >> 6) << 4)
    m[..., 4:8] = (S[..., 8:12] >> 4) | ((S[..., 4:8] >> 6) << 4)
    return sc, m


def q4k_fields(blocks: np.ndarray):
    """Fields of Q4_K super-blocks ``blocks[..., 144]``.

    Layout ([8e] §3.2, the q4_K kernel's reads): f16 ``d`` at byte 0, f16
    ``dmin`` at 2, 12 bytes of packed scales/mins at 4, 128 bytes of 4-bit
    values at 16.  Sub-block ``j`` (32 weights) takes its values from bytes
    ``16 + 32*(j // 2) + l`` -- the low nibble for even ``j``, the high nibble
    for odd ``j``.

    The 12 packed bytes ``S`` hold eight 6-bit scales ``sc`` and eight 6-bit
    mins ``m`` (reading: GGUF K-quant packing):
      j < 4:  sc_j = S[j] & 63,            m_j = S[j+4] & 63
      j >= 4: sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
              m_j  = (S[j+4] >> 4) | (S[j]   >> 6) << 4

    Returns ``d, dmin`` (float64 [...]), ``sc, m`` (int64 [..., 8]) and
    ``nib`` (int64 [..., 256]) in element order.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    if b.shape[-1] != Q4K_BYTES:
        raise ValueError("Q4_K blocks are 144 bytes")
    d = _f16_at(b, 0)
    dmin = _f16_at(b, 2)
    sc, m = _scales_mins(b[..., 4:16])
    qs = b[..., 16:144].astype(np.int64).reshape(b.shape[:-1] + (4, 32))  # [pair][l]
    lo = qs & 15          # sub-block 2*pair
    hi = qs >> 4          # sub-block 2*pair + 1
    nib = np.stack([lo, hi], axis=-2).reshape(b.shape[:-1] + (256,))
    return d, dmin, sc, m, nib


def q4k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Dequantised Q4_K weights: rows ``blocks[M, K/256, 144]`` -> float64 [M, K].

    Each weight is ``d * sc_j * nib - dmin * m_j`` ([8e] §2, the min-term
    paragraph).
    """
    d, dmin, sc, m, nib = q4k_fields(blocks)
    nib = nib.reshape(nib.shape[:-1] + (8, 32)).astype(np.float64)
    w = (d[..., None, None] * sc[..., :, None].astype(np.float64) * nib
         - dmin[..., None, None] * m[..., :, None].astype(np.float64))
    lead = blocks.shape[:-2]
    return w.reshape(lead + (blocks.shape[-2] * 256,))


def q5k_fields(blocks: np.ndarray):
    """Fields of Q5_K super-blocks ``blocks[..., 176]``.

    The pages name Q5_K as a third k-quant with matvec kernels of its own
    ([8e] §1 and §6) but do not give its layout.  Reading: GGUF's Q5_K --
    f16 ``d`` at byte 0, f16 ``dmin`` at 2, the 12 packed scale/min bytes of
    Q4_K at 4, ``qh[32]`` at 16, ``qs[128]`` at 48.  Sub-block ``j`` (32
    weights), lane ``l``: the low four bits are the nibble of
    ``qs[32*(j // 2) + l]`` (low for even ``j``, high for odd ``j``), bit four
    is bit ``j`` of ``qh[l]``; ``q5 = nib | hbit << 4`` (0..31).

    Returns ``d, dmin`` (float64 [...]), ``sc, m`` (int64 [..., 8]) and
    ``q5`` (int64 [..., 256]) in element order.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    if b.shape[-1] != Q5K_BYTES:
        raise ValueError("Q5_K blocks are 176 bytes")
    d = _f16_at(b, 0)
    dmin = _f16_at(b, 2)
    sc, m = _scales_mins(b[..., 4:16])
    qh = b[..., 16:48].astype(np.int64)                                    # [l]
    qs = b[..., 48:176].astype(np.int64).reshape(b.shape[:-1] + (4, 32))   # [pair][l]
    nib = np.stack([qs & 15, qs >> 4], axis=-2).reshape(b.shape[:-1] + (8, 32))  # [j][l]
    j = np.arange(8)[:, None]
    hbit = (qh[..., None, :] >> j) & 1                                     # [j][l]
    q5 = (nib | (hbit << 4)).reshape(b.shape[:-1] + (256,))
    return d, dmin, sc, m, q5


def q5k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Dequantised Q5_K weights ``d*sc_j*q5 - dmin*m_j``: [M, K/256, 176] -> float64 [M, K]."""
    d, dmin, sc, m, q5 = q5k_fields(blocks)
    q5 = q5.reshape(q5.shape[:-1] + (8, 32)).astype(np.float64)
    w = (d[..., None, None] * sc[..., :, None].astype(np.float64) * q5
         - dmin[..., None, None] * m[..., :, None].astype(np.float64))
    lead = blocks.shape[:-2]
    return w.reshape(lead + (blocks.shape[-2] * 256,))


# Q6_K element mapping (reading: GGUF).  Element e of a super-block lies in
# half h = e // 128; within it, group g = (e % 128) // 32 and lane l = e % 32.
_E = np.arange(256)
_H, _R = _E // 128, _E % 128
_G, _L = _R // 32, _R % 32
Q6K_QL_INDEX = 64 * _H + 32 * (_G & 1) + _L
Q6K_QL_SHIFT = 4 * (_G // 2)
Q6K_QH_INDEX = 32 * _H + _L
Q6K_QH_SHIFT = 2 * _G
Q6K_SC_INDEX = _E // 16


def q6k_fields(blocks: np.ndarray):
    """Fields of Q6_K super-blocks ``blocks[..., 210]``.

    Layout ([8e] §3.3, the generator pitfall): ``ql[128]`` at 0, ``qh[64]`` at
    128, int8 ``sc[16]`` at 192, f16 ``d`` at 208.  Each weight has a 6-bit
    value ``q6 = low4 | hi2 << 4`` with ``low4`` a nibble of ``ql`` and
    ``hi2`` a bit pair of ``qh`` (index tables above), and scale ``sc[e//16]``
    (16-weight sub-blocks, [8e] §3.1).

    Returns ``d`` (float64 [...]), ``sc`` (int64 [..., 16]) and ``q6``
    (int64 [..., 256], values 0..63).
    """
    b = np.asarray(blocks, dtype=np.uint8)
    if b.shape[-1] != Q6K_BYTES:
        raise ValueError("Q6_K blocks are 210 bytes")
    ql = b[..., 0:128].astype(np.int64)
    qh = b[..., 128:192].astype(np.int64)
    sc = np.ascontiguousarray(b[..., 192:208]).view(np.int8).astype(np.int64)
    d = _f16_at(b, 208)
    low4 = (ql[..., Q6K_QL_INDEX] >> Q6K_QL_SHIFT) & 15
    hi2 = (qh[..., Q6K_QH_INDEX] >> Q6K_QH_SHIFT) & 3
    q6 = low4 | (hi2 << 4)
    return d, sc, q6


def q6k_dequant(blocks: np.ndarray) -> np.ndarray:
    """Dequantised Q6_K weights ``d * sc[e//16] * (q6 - 32)``: [M, K/256, 210] -> float64 [M, K]."""
    d, sc, q6 = q6k_fields(blocks)
    w = d[..., None] * sc[..., Q6K_SC_INDEX].astype(np.float64) * (q6 - 32).astype(np.float64)
    lead = blocks.shape[:-2]
    return w.reshape(lead + (blocks.shape[-2] * 256,))


def q8_1_fields(xq: np.ndarray):
    """Fields of Q8_1 ("pad40") activation blocks ``xq[..., 40]``.

    Layout ([8e] §2 and the quantizer of §3.2): f16 ``d`` at 0, two pad bytes,
    32 int8 values at 4, int32 sum of those values at 36.  Returns ``d``
    (float64 [...]), ``q`` (int64 [..., 32]), ``pad`` (int64 [...]) and
    ``qsum`` (int64 [...]).
    """
    b = np.asarray(xq, dtype=np.uint8)
    if b.shape[-1] != Q8_1_BYTES:
        raise ValueError("Q8_1 blocks are 40 bytes")
    d = _f16_at(b, 0)
    pad = b[..., 2].astype(np.int64) | (b[..., 3].astype(np.int64) << 8)
    q = np.ascontiguousarray(b[..., 4:36]).view(np.int8).astype(np.int64)
    qsum = np.ascontiguousarray(b[..., 36:40]).view("<i4")[..., 0].astype(np.int64)
    return d, q, pad, qsum


def q8_1_dequant(xq: np.ndarray) -> np.ndarray:
    """Dequantised activations ``d16 * q``: ``xq[T, K/32, 40]`` -> float64 [T, K]."""
    d, q, _, _ = q8_1_fields(xq)
    x = d[..., None] * q.astype(np.float64)
    return x.reshape(xq.shape[:-2] + (xq.shape[-2] * 32,))
