"""Python binding of libqmm: fused-dequant Q4_K / Q5_K / Q6_K x Q8_1 matmul on MI355X.

Thin marshalling over the C ABI of ``include/qmm.h``: each function checks
tensor dtypes, devices and shapes, allocates outputs with torch, and passes
raw device pointers and the current HIP stream.  Every step of the
computation runs in the HIP kernels of ``libqmm.so``.

Tensor layouts (uint8 unless stated):
  Q4_K weights  [M, K/256, 144]      Q5_K weights  [M, K/256, 176]
  Q6_K weights  [M, K/256, 210]
  Q8_1 blocks   [rows, K/32, 40]     outputs       float32 [T, M]
  MoE experts   [E, M, K/256, bytes] (contiguous; the expert stride is taken
                from the tensor)
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    QMM_MMVQ_MAX_T, QMM_OP_MMQ, QMM_OP_MOE, QMM_OP_MOE_SLOTS, QMM_OP_MOE_FFN, QMM_Q4_K, QMM_Q5_K, QMM_Q6_K, QmmError, LIB_PATH,
)

__all__ = [
    "q8_1_quantize", "mmvq_q4k", "mmvq_q5k", "mmvq_q6k", "mmvq_pair", "mmq_q4k", "mmq_q5k", "mmq_q6k", "mmq_q4k_f32", "mmq_q5k_f32",
    "mmq_q6k_f32",
    "moe_grouped_mmq", "moe_grouped_swiglu", "moe_ffn", "moe_slot_mmvq",
    "swiglu_q8_1", "workspace", "workspace_bytes", "debug_subdots", "probe_read", "probe_read_geom",
    "probe_mfma", "probe_mfma_epilogue", "QmmError",
    "QMM_Q4_K", "QMM_Q5_K", "QMM_Q6_K", "LIB_PATH",
]

_BLOCK_BYTES = {QMM_Q4_K: 144, QMM_Q5_K: 176, QMM_Q6_K: 210}


def _p(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _out(out: torch.Tensor | None, shape: tuple, dtype: torch.dtype, device: torch.device, name: str = "out"):
    """A new output of ``shape``, or the caller's ``out`` checked to match it exactly.

    The C ABI cannot see buffer sizes, so a caller buffer of the wrong shape
    is rejected here before any device write."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(out, dtype, name, len(shape))
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.device != device:
        raise ValueError(f"{name} must be on {device}")
    return out


def _weights(w: torch.Tensor, fmt: int, name: str = "w"):
    _need(w, torch.uint8, name, 3)
    if w.shape[2] != _BLOCK_BYTES[fmt]:
        raise ValueError(f"{name}: blocks of {_BLOCK_BYTES[fmt]} bytes expected")
    return w.shape[0], w.shape[1] * 256


def _acts(xq: torch.Tensor, K: int, name: str = "xq"):
    _need(xq, torch.uint8, name, 3)
    if xq.shape[2] != 40 or xq.shape[1] * 32 != K:
        raise ValueError(f"{name}: expected [rows, {K // 32}, 40], got {tuple(xq.shape)}")
    return xq.shape[0]


def workspace_bytes(op: int, M: int = 0, K: int = 0, T: int = 0, E: int = 0, top_k: int = 0) -> int:
    return int(_lib.LIB.qmm_workspace_bytes(op, M, K, T, E, top_k))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace of ``nbytes`` bytes (16-byte multiple) on ``device``."""
    return torch.zeros((max(16, (nbytes + 15) // 16 * 16),), dtype=torch.uint8, device=device)


_MMQ_WS: dict = {}


def _mmq_ws(device: torch.device, M: int, K: int, T: int) -> torch.Tensor:
    """GEMM workspace cached per (device, current stream), grown to fit ``M``, ``K`` and ``T``.

    The workspace holds the call's queue counters, split-K arrival counters
    and repacked activations, so two calls may share one only if they are
    ordered on one stream: each stream gets its own.  A workspace is
    allocated while its stream is current, so the caching allocator reuses
    a replaced one only for work ordered after it on that stream (no
    synchronisation needed).  Pass ``ws`` explicitly to manage it yourself.
    """
    idx = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(device)
    key = (idx, stream.cuda_stream)
    need = workspace_bytes(QMM_OP_MMQ, M, K, T)
    ws = _MMQ_WS.get(key)
    if ws is None or ws.numel() < need:
        ws = workspace(need, device)
        _MMQ_WS[key] = ws
    return ws


def q8_1_quantize(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 ``x[T, K]`` -> Q8_1 blocks ``[T, K/32, 40]``."""
    _need(x, torch.float32, "x", 2)
    T, K = x.shape
    if K % 32:
        raise ValueError(f"x: K = {K} is not a multiple of 32")
    out = _out(out, (T, K // 32, 40), torch.uint8, x.device)
    _lib.call("q8_1_quantize", _p(x), _p(out), T, K, _stream(x.device))
    return out


def _mmvq(name: str, fmt: int, w, xq, out):
    M, K = _weights(w, fmt)
    T = _acts(xq, K)
    out = _out(out, (T, M), torch.float32, w.device)
    _lib.call(name, _p(w), _p(xq), _p(out), M, K, T, _stream(w.device))
    return out


def mmvq_q4k(w: torch.Tensor, xq: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode matvec, Q4_K weights x Q8_1 activations (T <= 8) -> fp32 [T, M]."""
    return _mmvq("mmvq_q4k", QMM_Q4_K, w, xq, out)


def mmvq_q5k(w: torch.Tensor, xq: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode matvec, Q5_K weights x Q8_1 activations (T <= 8) -> fp32 [T, M]."""
    return _mmvq("mmvq_q5k", QMM_Q5_K, w, xq, out)


def mmvq_q6k(w: torch.Tensor, xq: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode matvec, Q6_K weights x Q8_1 activations (T <= 8) -> fp32 [T, M]."""
    return _mmvq("mmvq_q6k", QMM_Q6_K, w, xq, out)


def mmvq_pair(fmt_a: int, wa: torch.Tensor, fmt_b: int, wb: torch.Tensor, xq: torch.Tensor,
              out_a: torch.Tensor | None = None, out_b: torch.Tensor | None = None):
    """Two one-token matvecs on the same Q8_1 row ``xq[1, K/32, 40]`` in one
    launch -> (fp32 [1, Ma], fp32 [1, Mb]), each bit-identical to the single
    matvec of its format."""
    Ma, K = _weights(wa, fmt_a, "wa")
    Mb, Kb = _weights(wb, fmt_b, "wb")
    if Kb != K:
        raise ValueError(f"wa and wb must have the same K, got {K} and {Kb}")
    if _acts(xq, K) != 1:
        raise ValueError("mmvq_pair takes one activation row")
    if wb.device != wa.device or xq.device != wa.device:
        raise ValueError("wa, wb and xq must be on one device")
    out_a = _out(out_a, (1, Ma), torch.float32, wa.device, "out_a")
    out_b = _out(out_b, (1, Mb), torch.float32, wa.device, "out_b")
    if out_a.data_ptr() == out_b.data_ptr():
        raise ValueError("out_a and out_b must be distinct")
    _lib.call("mmvq_pair", fmt_a, _p(wa), Ma, _p(out_a), fmt_b, _p(wb), Mb, _p(out_b), _p(xq), K,
              _stream(wa.device))
    return out_a, out_b


def _mmq(name: str, fmt: int, w, xq, out, ws):
    M, K = _weights(w, fmt)
    T = _acts(xq, K)
    out = _out(out, (T, M), torch.float32, w.device)
    ws = _mmq_ws(w.device, M, K, T) if ws is None else ws
    _need(ws, torch.uint8, "ws", 1)
    _lib.call(name, _p(w), _p(xq), _p(out), M, K, T, _p(ws), ws.numel(), _stream(w.device))
    return out


def mmq_q4k(w, xq, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM, Q4_K weights x Q8_1 activations -> fp32 [T, M] (int8 MFMA)."""
    return _mmq("mmq_q4k", QMM_Q4_K, w, xq, out, ws)


def mmq_q5k(w, xq, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM, Q5_K weights x Q8_1 activations -> fp32 [T, M] (int8 MFMA)."""
    return _mmq("mmq_q5k", QMM_Q5_K, w, xq, out, ws)


def mmq_q6k(w, xq, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM, Q6_K weights x Q8_1 activations -> fp32 [T, M] (int8 MFMA)."""
    return _mmq("mmq_q6k", QMM_Q6_K, w, xq, out, ws)


def _mmq_f32(name: str, fmt: int, w, x, out, ws):
    M, K = _weights(w, fmt)
    _need(x, torch.float32, "x", 2)
    if x.shape[1] != K:
        raise ValueError(f"x: expected [T, {K}], got {tuple(x.shape)}")
    T = x.shape[0]
    out = _out(out, (T, M), torch.float32, w.device)
    ws = _mmq_ws(w.device, M, K, T) if ws is None else ws
    _need(ws, torch.uint8, "ws", 1)
    _lib.call(name, _p(w), _p(x), _p(out), M, K, T, _p(ws), ws.numel(), _stream(w.device))
    return out


def mmq_q4k_f32(w, x, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM with fp32 activations ``x[T, K]`` quantized to Q8_1 inside the call."""
    return _mmq_f32("mmq_q4k_f32", QMM_Q4_K, w, x, out, ws)


def mmq_q5k_f32(w, x, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM with fp32 activations ``x[T, K]`` quantized to Q8_1 inside the call."""
    return _mmq_f32("mmq_q5k_f32", QMM_Q5_K, w, x, out, ws)


def mmq_q6k_f32(w, x, out=None, ws=None) -> torch.Tensor:
    """Prefill GEMM with fp32 activations ``x[T, K]`` quantized to Q8_1 inside the call."""
    return _mmq_f32("mmq_q6k_f32", QMM_Q6_K, w, x, out, ws)


def moe_grouped_mmq(fmt: int, w: torch.Tensor, xq: torch.Tensor, ids: torch.Tensor,
                    expert_weights: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, reuse_routing: bool = False) -> torch.Tensor:
    """Grouped expert GEMM.

    ``w`` [E, M, K/256, bytes]; ``ids`` int32 [T, top_k]; ``xq`` has T rows
    (one per token) or T*top_k rows (one per slot).  Without
    ``expert_weights`` the result is per slot, [T*top_k, M]; with fp32
    ``expert_weights`` [T, top_k] it is the weighted sum over k, [T, M].

    ``reuse_routing`` calls ``moe_grouped_mmq_routed``: the route tables that
    the previous grouped call on ``ws`` (same ``ids``, T, top_k and E, issued
    earlier on the current stream) left in ``ws`` are used instead of being
    prepared again; ``ws`` must then be given and large enough for this call.
    """
    _need(w, torch.uint8, "w", 4)
    if w.shape[3] != _BLOCK_BYTES[fmt]:
        raise ValueError("w: wrong block size for fmt")
    E, M, K = w.shape[0], w.shape[1], w.shape[2] * 256
    _need(ids, torch.int32, "ids", 2)
    T, top_k = ids.shape
    rows = _acts(xq, K)
    if rows == T:
        rows_per_token = 1
    elif rows == T * top_k:
        rows_per_token = top_k
    else:
        raise ValueError("xq must have T or T*top_k rows")
    if expert_weights is not None:
        _need(expert_weights, torch.float32, "expert_weights", 2)
        if tuple(expert_weights.shape) != (T, top_k):
            raise ValueError("expert_weights must be [T, top_k]")
    out_rows = T if expert_weights is not None else T * top_k
    out = _out(out, (out_rows, M), torch.float32, w.device)
    need = workspace_bytes(QMM_OP_MOE if expert_weights is not None else QMM_OP_MOE_SLOTS, M, K, T, E, top_k)
    if ws is None:
        if reuse_routing:
            raise ValueError("reuse_routing needs the workspace of the call that prepared the routing")
        ws = workspace(need, w.device)
    _need(ws, torch.uint8, "ws", 1)
    stride = w.stride(0)
    _lib.call("moe_grouped_mmq_routed" if reuse_routing else "moe_grouped_mmq", fmt, _p(w), E, M, K, stride,
              _p(xq), rows_per_token, _p(ids), _p(expert_weights), T, top_k, _p(out), _p(ws), ws.numel(),
              _stream(w.device))
    return out


def moe_grouped_swiglu(fmt: int, w: torch.Tensor, xq: torch.Tensor, ids: torch.Tensor,
                       out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped gate||up product with SwiGLU -> Q8_1 fused: ``w`` [E, 2F, K/256, bytes]
    (gate rows then up rows per expert) -> Q8_1 ``[T*top_k, F/32, 40]``, the bytes
    of :func:`moe_grouped_mmq` (per slot) followed by :func:`swiglu_q8_1`.  The
    route tables it leaves in ``ws`` serve a following ``reuse_routing`` call."""
    _need(w, torch.uint8, "w", 4)
    if w.shape[3] != _BLOCK_BYTES[fmt]:
        raise ValueError("w: wrong block size for fmt")
    E, M, K = w.shape[0], w.shape[1], w.shape[2] * 256
    if M % 256:
        raise ValueError(f"w: 2F = {M} rows per expert must be a multiple of 256")
    _need(ids, torch.int32, "ids", 2)
    T, top_k = ids.shape
    rows = _acts(xq, K)
    if rows == T:
        rows_per_token = 1
    elif rows == T * top_k:
        rows_per_token = top_k
    else:
        raise ValueError("xq must have T or T*top_k rows")
    out = _out(out, (T * top_k, M // 64, 40), torch.uint8, w.device)
    need = workspace_bytes(QMM_OP_MOE_SLOTS, M, K, T, E, top_k)
    ws = workspace(need, w.device) if ws is None else ws
    _need(ws, torch.uint8, "ws", 1)
    _lib.call("moe_grouped_mmq_swiglu", fmt, _p(w), E, M, K, w.stride(0), _p(xq), rows_per_token, _p(ids), T, top_k,
              _p(out), _p(ws), ws.numel(), _stream(w.device))
    return out


def moe_ffn(fmt_gu: int, w_gu: torch.Tensor, fmt_dn: int, w_dn: torch.Tensor, xq: torch.Tensor, ids: torch.Tensor,
            expert_weights: torch.Tensor, out: torch.Tensor | None = None,
            ws: torch.Tensor | None = None) -> torch.Tensor:
    """A routed FFN layer in one call: ``w_gu`` [E, 2F, H/256, bytes] (gate rows
    then up rows), ``w_dn`` [E, H, F/256, bytes], ``xq`` Q8_1 [T, H/32, 40],
    ``ids`` int32 and ``expert_weights`` fp32 [T, top_k] -> fp32 [T, H]; the bits
    of :func:`moe_grouped_swiglu` followed by the weighted routed down call."""
    _need(w_gu, torch.uint8, "w_gu", 4)
    _need(w_dn, torch.uint8, "w_dn", 4)
    if w_gu.shape[3] != _BLOCK_BYTES[fmt_gu] or w_dn.shape[3] != _BLOCK_BYTES[fmt_dn]:
        raise ValueError("w_gu / w_dn: wrong block size for the format")
    E, F2, H = w_gu.shape[0], w_gu.shape[1], w_gu.shape[2] * 256
    F = F2 // 2
    if F2 % 512 or w_dn.shape[0] != E or w_dn.shape[1] != H or w_dn.shape[2] * 256 != F:
        raise ValueError(f"expected w_gu [E, 2F, H/256] and w_dn [E, H, F/256] with F % 256 == 0, got "
                         f"{tuple(w_gu.shape)} and {tuple(w_dn.shape)}")
    _need(ids, torch.int32, "ids", 2)
    T, top_k = ids.shape
    if _acts(xq, H) != T:
        raise ValueError("xq must have one row per token")
    _need(expert_weights, torch.float32, "expert_weights", 2)
    if tuple(expert_weights.shape) != (T, top_k):
        raise ValueError("expert_weights must be [T, top_k]")
    out = _out(out, (T, H), torch.float32, w_gu.device)
    need = workspace_bytes(QMM_OP_MOE_FFN, H, F, T, E, top_k)
    ws = workspace(need, w_gu.device) if ws is None else ws
    _need(ws, torch.uint8, "ws", 1)
    _lib.call("moe_ffn", fmt_gu, _p(w_gu), w_gu.stride(0), fmt_dn, _p(w_dn), w_dn.stride(0), E, H, F, _p(xq), _p(ids),
              _p(expert_weights), T, top_k, _p(out), _p(ws), ws.numel(), _stream(w_gu.device))
    return out


def moe_slot_mmvq(fmt: int, w: torch.Tensor, xq: torch.Tensor, ids: torch.Tensor,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-slot expert matvec (the path the grouped GEMM replaces).

    Same layouts as :func:`moe_grouped_mmq` without ``expert_weights``:
    result [T*top_k, M], row t*top_k + k = W[ids[t, k]] . x_row.
    """
    _need(w, torch.uint8, "w", 4)
    if w.shape[3] != _BLOCK_BYTES[fmt]:
        raise ValueError("w: wrong block size for fmt")
    E, M, K = w.shape[0], w.shape[1], w.shape[2] * 256
    _need(ids, torch.int32, "ids", 2)
    T, top_k = ids.shape
    rows = _acts(xq, K)
    if rows == T:
        rows_per_token = 1
    elif rows == T * top_k:
        rows_per_token = top_k
    else:
        raise ValueError("xq must have T or T*top_k rows")
    out = _out(out, (T * top_k, M), torch.float32, w.device)
    _lib.call("moe_slot_mmvq", fmt, _p(w), E, M, K, w.stride(0), _p(xq), rows_per_token, _p(ids), T, top_k,
              _p(out), _stream(w.device))
    return out


def swiglu_q8_1(g_u: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows ``g_u[R, 2F]`` (gate | up) -> Q8_1 of silu(gate) * up, ``[R, F/32, 40]``."""
    _need(g_u, torch.float32, "g_u", 2)
    R, F2 = g_u.shape
    if F2 % 64:
        raise ValueError(f"g_u: width {F2} must be 2*F with F a multiple of 32")
    F = F2 // 2
    out = _out(out, (R, F // 32, 40), torch.uint8, g_u.device)
    _lib.call("swiglu_q8_1", _p(g_u), _p(out), R, F, _stream(g_u.device))
    return out


def debug_subdots(fmt: int, path: int, w: torch.Tensor, xq: torch.Tensor):
    """Integer stage of the MMVQ (path 0) or MMQ (path 1) kernel: (D, S) int32.

    Q4_K, Q5_K: D [T, M, K/32], S [T, K/32]; Q6_K: D [T, M, K/16], S None.
    """
    M, K = _weights(w, fmt)
    T = _acts(xq, K)
    nsub = K // 16 if fmt == QMM_Q6_K else K // 32
    D = torch.empty((T, M, nsub), dtype=torch.int32, device=w.device)
    S = torch.empty((T, K // 32), dtype=torch.int32, device=w.device) if fmt != QMM_Q6_K else None
    ws = _mmq_ws(w.device, M, K, T)
    _lib.call("qmm_debug_subdots", fmt, path, _p(w), _p(xq), _p(D), _p(S), M, K, T, _p(ws),
              ws.numel(), _stream(w.device))
    return D, S


def probe_read(buf: torch.Tensor, nbytes: int | None = None, sink: torch.Tensor | None = None):
    """Enqueue the read-only ceiling probe over the first ``nbytes`` of ``buf``."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if sink is None:
        sink = torch.zeros((4,), dtype=torch.int32, device=buf.device)
    _lib.call("qmm_probe_read", _p(buf), nbytes, _p(sink), _stream(buf.device))
    return sink


def probe_read_geom(buf: torch.Tensor, nbytes: int, loads_per_thread: int, grid: int = 0,
                    sink: torch.Tensor | None = None):
    """Enqueue the read probe with ``loads_per_thread`` loads in flight per thread and ``grid``
    workgroups (0: one pass)."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink is None:
        sink = torch.zeros((4,), dtype=torch.int32, device=buf.device)
    _lib.call("qmm_probe_read_geom", _p(buf), nbytes, loads_per_thread, grid, _p(sink), _stream(buf.device))
    return sink


def probe_mfma(iters: int, waves_per_simd: int, sink: torch.Tensor) -> torch.Tensor:
    """Enqueue the int8-MFMA-only probe (see include/qmm.h for its op count)."""
    _need(sink, torch.int32, "sink", 1)
    _lib.call("qmm_probe_mfma", iters, waves_per_simd, _p(sink), _stream(sink.device))
    return sink


def probe_mfma_epilogue(mode: int, iters: int, waves_per_simd: int, sink: torch.Tensor) -> torch.Tensor:
    """Enqueue the MFMA + fp32 epilogue probe (mode 1, 2 or 3; see include/qmm.h)."""
    _need(sink, torch.int32, "sink", 1)
    _lib.call("qmm_probe_mfma_epilogue", mode, iters, waves_per_simd, _p(sink), _stream(sink.device))
    return sink
