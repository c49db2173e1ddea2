"""ctypes loader for the in-tree ``libqmm.so`` and its C ABI (``include/qmm.h``).

torch is imported first so that its HIP runtime (soname ``libamdhip64.so.7``)
is the one libqmm binds to: device pointers and streams are then shared.
There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libqmm links against)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmm.so")

QMM_OK = 0
QMM_ERR_NULL = -1
QMM_ERR_SHAPE = -2
QMM_ERR_ALIGN = -3
QMM_ERR_WORKSPACE = -4
QMM_ERR_HIP = -5
QMM_ERR_UNSUPPORTED = -6
QMM_ERR_SCRATCH = -7
QMM_STATIC_SCRATCH_BYTES = 32 << 20
QMM_Q4_K = 12
QMM_Q5_K = 13
QMM_Q6_K = 14
QMM_OP_MMQ = 1
QMM_OP_MOE = 2
QMM_OP_MOE_SLOTS = 3
QMM_OP_MOE_FFN = 4
QMM_MMVQ_MAX_T = 8

_vp, _i64, _sz, _i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int

# name -> (restype, argtypes); every symbol declared in include/qmm.h
SIGNATURES = {
    "q8_1_quantize": (_i, [_vp, _vp, _i64, _i64, _vp]),
    "mmvq_q4k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "mmvq_q5k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "mmvq_q6k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "mmvq_pair": (_i, [_i, _vp, _i64, _vp, _i, _vp, _i64, _vp, _vp, _i64, _vp]),
    "mmq_q4k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "mmq_q5k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "mmq_q6k": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "mmq_q4k_noalloc": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "mmq_q4k_f32": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "mmq_q5k_f32": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "mmq_q6k_f32": (_i, [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "moe_grouped_mmq": (_i, [_i, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _i64,
                             _vp, _vp, _sz, _vp]),
    "moe_ffn": (_i, [_i, _vp, _i64, _i, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "moe_grouped_mmq_swiglu": (_i, [_i, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _sz,
                                    _vp]),
    "moe_grouped_mmq_routed": (_i, [_i, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _i64,
                                    _vp, _vp, _sz, _vp]),
    "moe_slot_mmvq": (_i, [_i, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _vp]),
    "swiglu_q8_1": (_i, [_vp, _vp, _i64, _i64, _vp]),
    "qmm_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i64, _i64]),
    "qmm_workspace_init": (_i, [_vp, _sz, _vp]),
    "qmm_status_str": (ctypes.c_char_p, [_i]),
    "qmm_debug_subdots": (_i, [_i, _i, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "qmm_probe_read": (_i, [_vp, _sz, _vp, _vp]),
    "qmm_probe_mfma": (_i, [_i64, _i, _vp, _vp]),
    "qmm_probe_mfma_epilogue": (_i, [_i, _i64, _i, _vp, _vp]),
    "qmm_probe_read_geom": (_i, [_vp, _sz, _i, _i64, _vp, _vp]),
}


class QmmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = LIB.qmm_status_str(status).decode() if LIB is not None else str(status)
        super().__init__(f"{fn} failed with status {status} ({msg})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with quantized_matmul_q8_amd/build.py "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = None
LIB = _load()


def call(name: str, *args) -> None:
    st = getattr(LIB, name)(*args)
    if st != QMM_OK:
        raise QmmError(name, st)
