"""C ABI checks that need no GPU: the library loads, exports every function that
include/qmm.h declares, and rejects bad arguments on the host with the
documented status codes before anything is enqueued.

Every call below fails host validation, so no kernel is launched and the
fake (aligned, non-null) device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

qmm = pytest.importorskip("quantized_matmul_q8_amd")
from quantized_matmul_q8_amd import _lib  # noqa: E402

L = _lib.LIB
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
MISAL = ctypes.c_void_p(0x10004)     # 4-byte aligned only
NUL = ctypes.c_void_p(0)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("q8_1_quantize", "mmvq_q4k", "mmvq_q6k", "mmq_q4k", "mmq_q6k", "mmq_q4k_f32", "mmq_q6k_f32",
              "moe_grouped_mmq"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.SIGNATURES) == names


def test_library_is_in_tree():
    assert os.path.dirname(os.path.abspath(_lib.LIB_PATH)) == os.path.join(ROOT, "quantized_matmul_q8_amd")


def test_status_strings():
    assert L.qmm_status_str(0) == b"ok"
    for st in range(-7, 0):
        assert L.qmm_status_str(st) not in (b"ok", b"unknown status")
    assert L.qmm_status_str(-99) == b"unknown status"


def test_workspace_sizes():
    assert L.qmm_workspace_bytes(_lib.QMM_OP_MMQ, 4096, 4096, 512, 0, 0) >= 36
    # few tiles (4096 rows, 8 tokens): room for the fp32 partial tiles of the K splits
    small = L.qmm_workspace_bytes(_lib.QMM_OP_MMQ, 4096, 11008, 8, 0, 0)
    assert small >= 43 * 12288 + 32 * 2 * 16384
    # one row block with many tokens needs no partials: the size grows only with T
    assert L.qmm_workspace_bytes(_lib.QMM_OP_MMQ, 4096, 4096, 512, 0, 0) < 2048 + 16 * 16 * 12288 + 256
    moe = L.qmm_workspace_bytes(_lib.QMM_OP_MOE, 2048, 768, 512, 128, 8)
    # per-slot fp32 scratch dominates: T*top_k*M*4
    assert moe >= 512 * 8 * 2048 * 4
    assert L.qmm_workspace_bytes(99, 1, 1, 1, 1, 1) == 0


def test_quantize_errors():
    assert L.q8_1_quantize(FAKE, FAKE, 1, 33, NUL) == _lib.QMM_ERR_SHAPE
    assert L.q8_1_quantize(FAKE, FAKE, -1, 32, NUL) == _lib.QMM_ERR_SHAPE
    assert L.q8_1_quantize(NUL, FAKE, 1, 32, NUL) == _lib.QMM_ERR_NULL
    assert L.q8_1_quantize(MISAL, FAKE, 1, 32, NUL) == _lib.QMM_ERR_ALIGN
    assert L.q8_1_quantize(NUL, NUL, 0, 32, NUL) == _lib.QMM_OK      # T = 0 is a no-op


@pytest.mark.parametrize("fn", ["mmvq_q4k", "mmvq_q5k", "mmvq_q6k"])
def test_mmvq_errors(fn):
    f = getattr(L, fn)
    assert f(FAKE, FAKE, FAKE, 4, 300, 1, NUL) == _lib.QMM_ERR_SHAPE     # K % 256
    assert f(FAKE, FAKE, FAKE, 4, 256, 9, NUL) == _lib.QMM_ERR_SHAPE     # T > 8
    assert f(FAKE, FAKE, FAKE, 0, 256, 1, NUL) == _lib.QMM_ERR_SHAPE     # M < 1
    assert f(FAKE, NUL, FAKE, 4, 256, 1, NUL) == _lib.QMM_ERR_NULL
    assert f(FAKE, FAKE, MISAL, 4, 256, 1, NUL) == _lib.QMM_ERR_ALIGN


def test_moe_swiglu_errors():
    f, Q4, Q6 = L.moe_grouped_mmq_swiglu, _lib.QMM_Q4_K, _lib.QMM_Q6_K
    big = ctypes.c_size_t(1 << 40)
    # fmt, w, E, M, K, stride, xq, rows_per_token, ids, T, top_k, hq, ws, ws_bytes, stream
    assert f(Q6, FAKE, 4, 256, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert f(Q4, FAKE, 4, 128, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_SHAPE
    assert f(Q4, FAKE, 4, 384, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_SHAPE
    assert f(Q4, FAKE, 4, 256, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, NUL, FAKE, big, NUL) == _lib.QMM_ERR_NULL
    assert f(Q4, FAKE, 4, 256, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, MISAL, FAKE, big, NUL) == _lib.QMM_ERR_ALIGN
    assert f(Q4, FAKE, 4, 256, 256, 1 << 20, FAKE, 1, FAKE, 8, 2, FAKE, FAKE, 16, NUL) == _lib.QMM_ERR_WORKSPACE


def test_moe_ffn_errors():
    f, Q4, Q6 = L.moe_ffn, _lib.QMM_Q4_K, _lib.QMM_Q6_K
    big = ctypes.c_size_t(1 << 40)
    S = 1 << 24
    # fmt_gu, w_gu, stride_gu, fmt_dn, w_dn, stride_dn, E, H, F, xq, ids, p, T, top_k, y, ws, ws_bytes, stream
    assert f(Q6, FAKE, S, Q4, FAKE, S, 4, 512, 256, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, big, NUL) == \
        _lib.QMM_ERR_UNSUPPORTED
    assert f(Q4, FAKE, S, 9, FAKE, S, 4, 512, 256, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, big, NUL) == \
        _lib.QMM_ERR_UNSUPPORTED
    assert f(Q4, FAKE, S, Q4, FAKE, S, 4, 512, 128, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_SHAPE
    assert f(Q4, FAKE, S, Q4, FAKE, S, 4, 500, 256, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_SHAPE
    assert f(Q4, FAKE, 16, Q4, FAKE, S, 4, 512, 256, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_SHAPE
    assert f(Q4, FAKE, S, Q4, FAKE, S, 4, 512, 256, FAKE, FAKE, NUL, 8, 2, FAKE, FAKE, big, NUL) == _lib.QMM_ERR_NULL
    assert f(Q4, FAKE, S, Q4, FAKE, S, 4, 512, 256, FAKE, FAKE, FAKE, 8, 2, MISAL, FAKE, big, NUL) == _lib.QMM_ERR_ALIGN
    assert f(Q4, FAKE, S, Q4, FAKE, S, 4, 512, 256, FAKE, FAKE, FAKE, 8, 2, FAKE, FAKE, 64, NUL) == \
        _lib.QMM_ERR_WORKSPACE
    assert L.qmm_workspace_bytes(_lib.QMM_OP_MOE_FFN, 2048, 768, 512, 128, 8) > \
        L.qmm_workspace_bytes(_lib.QMM_OP_MOE, 2048, 768, 512, 128, 8)


def test_mmvq_pair_errors():
    f, Q4, Q6 = L.mmvq_pair, _lib.QMM_Q4_K, _lib.QMM_Q6_K
    assert f(99, FAKE, 4, FAKE, Q4, FAKE, 4, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert f(Q4, FAKE, 4, FAKE, 7, FAKE, 4, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert f(Q4, FAKE, 4, FAKE, Q6, FAKE, 4, FAKE, FAKE, 300, NUL) == _lib.QMM_ERR_SHAPE     # K % 256
    assert f(Q4, FAKE, 0, FAKE, Q6, FAKE, 4, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_SHAPE     # Ma < 1
    assert f(Q4, FAKE, 4, FAKE, Q6, FAKE, 0, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_SHAPE     # Mb < 1
    assert f(Q4, FAKE, 4, FAKE, Q6, NUL, 4, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_NULL
    assert f(Q4, FAKE, 4, FAKE, Q6, FAKE, 4, FAKE, NUL, 256, NUL) == _lib.QMM_ERR_NULL
    assert f(Q4, FAKE, 4, MISAL, Q6, FAKE, 4, FAKE, FAKE, 256, NUL) == _lib.QMM_ERR_ALIGN


@pytest.mark.parametrize("fn", ["mmq_q4k", "mmq_q5k", "mmq_q6k", "mmq_q4k_f32", "mmq_q5k_f32", "mmq_q6k_f32"])
def test_mmq_errors(fn):
    f = getattr(L, fn)
    assert f(FAKE, FAKE, FAKE, 4, 256, 0, FAKE, 256, NUL) == _lib.QMM_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 255, 1, FAKE, 256, NUL) == _lib.QMM_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 256, 1, NUL, 256, NUL) == _lib.QMM_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 4, 256, 1, MISAL, 256, NUL) == _lib.QMM_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 256, 1, FAKE, 8, NUL) == _lib.QMM_ERR_WORKSPACE


@pytest.mark.parametrize("entry", ["moe_grouped_mmq", "moe_grouped_mmq_routed"])
def test_moe_errors(entry):
    f = getattr(L, entry)
    ok = dict(fmt=_lib.QMM_Q4_K, w=FAKE, E=8, M=64, K=256, stride=64 * 144, xq=FAKE, rpt=1,
              ids=FAKE, p=NUL, T=4, top_k=2, y=FAKE, ws=FAKE, wsb=16, st=NUL)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["fmt"], a["w"], a["E"], a["M"], a["K"], a["stride"], a["xq"], a["rpt"], a["ids"],
                 a["p"], a["T"], a["top_k"], a["y"], a["ws"], a["wsb"], a["st"])

    assert call(fmt=7) == _lib.QMM_ERR_UNSUPPORTED
    assert call(top_k=9) == _lib.QMM_ERR_SHAPE           # top_k > E
    assert call(rpt=3) == _lib.QMM_ERR_SHAPE             # rows per token not 1 or top_k
    assert call(stride=64 * 144 - 16) == _lib.QMM_ERR_SHAPE
    assert call(stride=64 * 144 + 8) == _lib.QMM_ERR_SHAPE      # Q4_K stride % 16
    assert call(fmt=_lib.QMM_Q6_K, stride=64 * 210 + 1) == _lib.QMM_ERR_SHAPE   # Q6_K stride % 2
    assert call(E=0) == _lib.QMM_ERR_SHAPE
    assert call(E=513, top_k=2) == _lib.QMM_ERR_SHAPE
    assert call(ids=NUL) == _lib.QMM_ERR_NULL
    assert call(p=MISAL) == _lib.QMM_ERR_ALIGN
    assert call() == _lib.QMM_ERR_WORKSPACE              # 16 bytes is too small


def test_slot_mmvq_errors():
    f = L.moe_slot_mmvq
    ok = dict(fmt=_lib.QMM_Q4_K, w=FAKE, E=8, M=64, K=256, stride=64 * 144, xq=FAKE, rpt=1,
              ids=FAKE, T=4, top_k=2, y=FAKE, st=NUL)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["fmt"], a["w"], a["E"], a["M"], a["K"], a["stride"], a["xq"], a["rpt"], a["ids"],
                 a["T"], a["top_k"], a["y"], a["st"])

    assert call(fmt=7) == _lib.QMM_ERR_UNSUPPORTED
    assert call(top_k=9) == _lib.QMM_ERR_SHAPE
    assert call(rpt=3) == _lib.QMM_ERR_SHAPE
    assert call(K=300) == _lib.QMM_ERR_SHAPE
    assert call(stride=64 * 144 + 8) == _lib.QMM_ERR_SHAPE
    assert call(T=40000, top_k=2) == _lib.QMM_ERR_SHAPE      # more than 65535 slots
    assert call(ids=NUL) == _lib.QMM_ERR_NULL
    assert call(y=MISAL) == _lib.QMM_ERR_ALIGN


def test_debug_and_probe_errors():
    f = L.qmm_debug_subdots
    assert f(3, 0, FAKE, FAKE, FAKE, FAKE, 4, 256, 1, FAKE, 256, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert f(_lib.QMM_Q4_K, 2, FAKE, FAKE, FAKE, FAKE, 4, 256, 1, FAKE, 256, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert f(_lib.QMM_Q4_K, 0, FAKE, FAKE, FAKE, FAKE, 4, 256, 9, FAKE, 256, NUL) == _lib.QMM_ERR_SHAPE
    assert f(_lib.QMM_Q4_K, 0, FAKE, FAKE, FAKE, NUL, 4, 256, 1, FAKE, 256, NUL) == _lib.QMM_ERR_NULL
    assert f(_lib.QMM_Q4_K, 1, FAKE, FAKE, FAKE, FAKE, 4, 256, 1, FAKE, 8, NUL) == _lib.QMM_ERR_WORKSPACE
    assert L.qmm_probe_read(FAKE, 20, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_read(NUL, 16, FAKE, NUL) == _lib.QMM_ERR_NULL
    assert L.swiglu_q8_1(FAKE, FAKE, 1, 48, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_workspace_init(MISAL, 16, NUL) == _lib.QMM_ERR_ALIGN


def test_mmq_limits_accepted_and_rejected_on_the_host():
    # sizes at the documented limits pass the shape checks (the NULL
    # workspace is reported next); one past them is a shape error
    f = L.mmq_q4k
    assert f(FAKE, FAKE, FAKE, 128, 256, 1 << 24, NUL, 0, NUL) == _lib.QMM_ERR_NULL      # T = 2^24
    assert f(FAKE, FAKE, FAKE, 128, 256, (1 << 24) + 1, NUL, 0, NUL) == _lib.QMM_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 128, 256 << 16, 64, NUL, 0, NUL) == _lib.QMM_ERR_NULL     # K/256 = 2^16
    assert f(FAKE, FAKE, FAKE, 128, 256 << 17, 64, NUL, 0, NUL) == _lib.QMM_ERR_SHAPE
    # output tiles: 2^14 row tiles x 2^18 column tiles = 2^32 > 2^30
    assert f(FAKE, FAKE, FAKE, 1 << 21, 256, 1 << 24, NUL, 0, NUL) == _lib.QMM_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 1 << 19, 256, 1 << 24, NUL, 0, NUL) == _lib.QMM_ERR_NULL   # 2^12 x 2^18 = 2^30
    # the workspace of a call with many column tiles is sized for every chunk
    # (the repack grid is launched in pieces of at most 65535 column tiles)
    T = 65535 * 32 + 100
    assert L.qmm_workspace_bytes(_lib.QMM_OP_MMQ, 128, 256, T, 0, 0) >= 2048 + ((T + 31) // 32) * 12288


def test_moe_limits_and_workspace_ops():
    f = L.moe_grouped_mmq

    def call(T, top_k, E=8, M=64, K=256, ws=NUL, wsb=0, p=NUL):
        return f(_lib.QMM_Q4_K, FAKE, E, M, K, M * (K // 256) * 144, FAKE, 1, FAKE, p, T, top_k, FAKE, ws, wsb, NUL)

    assert call(1 << 27, 8) == _lib.QMM_ERR_NULL                   # T*top_k = 2^30 slots
    assert call((1 << 27) + 1, 8) == _lib.QMM_ERR_SHAPE
    assert call(4, 2, K=256 << 17) == _lib.QMM_ERR_SHAPE           # K/256 > 2^16
    # work entries: ceil(M/128) x (slots + 31*min(E, slots))/32 > 2^30
    assert call(1 << 22, 8, M=128 * 1024) == _lib.QMM_ERR_SHAPE
    w = L.qmm_workspace_bytes
    slots = L.qmm_workspace_bytes(_lib.QMM_OP_MOE_SLOTS, 2048, 768, 512, 128, 8)
    weighted = w(_lib.QMM_OP_MOE, 2048, 768, 512, 128, 8)
    assert weighted - slots >= 512 * 8 * 2048 * 4         # the per-slot fp32 scratch
    assert slots < 512 * 8 * 2048 * 4
    # one token routed to 8 of 512 experts: at most 8 column tiles are repacked
    one = w(_lib.QMM_OP_MOE_SLOTS, 2048, 2048, 1, 512, 8)
    assert one <= 256 + 4 * (512 + 3 * 513 + 8) + 1024 + 8 * 8 * 12288 + 256
    # a weighted call rejects the per-slot size (no launch: the check fails)
    assert call(4, 2, ws=FAKE, wsb=w(_lib.QMM_OP_MOE_SLOTS, 64, 256, 4, 8, 2), p=FAKE) == _lib.QMM_ERR_WORKSPACE


def test_noalloc_host_errors():
    f = L.mmq_q4k_noalloc
    assert f(FAKE, FAKE, FAKE, 4, 256, 0, NUL) == _lib.QMM_ERR_SHAPE
    assert f(NUL, FAKE, FAKE, 4, 256, 1, NUL) == _lib.QMM_ERR_NULL
    assert f(FAKE, FAKE, MISAL, 4, 256, 1, NUL) == _lib.QMM_ERR_ALIGN
    # 1M tokens need gigabytes of workspace: refused before anything runs
    assert f(FAKE, FAKE, FAKE, 4096, 4096, 1 << 20, NUL) == _lib.QMM_ERR_SCRATCH
    assert L.qmm_status_str(_lib.QMM_ERR_SCRATCH) != b"unknown status"


def test_probe_hooks_host_errors():
    assert L.qmm_probe_mfma(0, 2, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_mfma(10, 3, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_mfma(10, 2, NUL, NUL) == _lib.QMM_ERR_NULL
    assert L.qmm_probe_mfma(10, 2, MISAL, NUL) == _lib.QMM_ERR_ALIGN
    assert L.qmm_probe_mfma_epilogue(10, 10, 2, FAKE, NUL) == _lib.QMM_ERR_UNSUPPORTED
    assert L.qmm_probe_mfma_epilogue(1, (1 << 24) + 1, 2, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_mfma_epilogue(1, 10, 8, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_read_geom(FAKE, 32, 3, 0, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_read_geom(FAKE, 20, 4, 0, FAKE, NUL) == _lib.QMM_ERR_SHAPE
    assert L.qmm_probe_read_geom(NUL, 32, 4, 0, FAKE, NUL) == _lib.QMM_ERR_NULL
