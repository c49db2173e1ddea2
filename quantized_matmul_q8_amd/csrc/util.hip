// Library-wide entry points: status text, workspace sizing and zero-fill,
// the debug integer-stage hook and the read-ceiling probe.
#include "qmm_common.hpp"

namespace qmm {

size_t moe_workspace_bytes(int64_t M, int64_t K, int64_t T, int64_t E, int64_t top_k, bool weighted);
size_t moe_ffn_workspace_bytes(int64_t H, int64_t F, int64_t T, int64_t E, int64_t top_k);
size_t mmq_workspace_bytes(int64_t M, int64_t K, int64_t T);
int debug_mmvq(int fmt, const void* w, const void* xq, int32_t* D, int32_t* S, int64_t M, int64_t K,
               int64_t T, hipStream_t st);
int mmq_dense(int fmt, const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
              void* ws, hipStream_t st, int32_t* dbgD, int32_t* dbgS, const float* xf);

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

static int zero_fill(void* p, size_t bytes, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(bytes / 4);
  if (n == 0) return QMM_OK;
  int64_t grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), n);
  return launch_status();
}

// Read-only streaming: every thread first issues all of its kProbeUnroll
// 16-byte loads (lane-contiguous, one grid stride apart), then folds them
// with xor, so each wave has kProbeUnroll loads in flight instead of one.
// The store is taken only for an improbable value, so the kernel writes
// (almost) nothing while the compiler must still perform every load.
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint4 v[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) {
    const int64_t i = i0 + u * stride;
    v[u] = i < n ? ld16_nt(p + i) : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace qmm

using namespace qmm;

extern "C" const char* qmm_status_str(int status) {
  switch (status) {
    case QMM_OK: return "ok";
    case QMM_ERR_NULL: return "null pointer argument";
    case QMM_ERR_SHAPE: return "size out of range or not a block multiple";
    case QMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMM_ERR_WORKSPACE: return "workspace too small";
    case QMM_ERR_HIP: return "HIP runtime error";
    case QMM_ERR_UNSUPPORTED: return "unsupported format or operation";
    case QMM_ERR_SCRATCH: return "call needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

extern "C" size_t qmm_workspace_bytes(int op, int64_t M, int64_t K, int64_t T, int64_t E,
                                      int64_t top_k) {
  if (M < 0 || K < 0 || T < 0 || E < 0 || top_k < 0) return 0;
  if (op == QMM_OP_MMQ) return mmq_workspace_bytes(M, K, T);
  if (op == QMM_OP_MOE) return moe_workspace_bytes(M, K, T, E, top_k, true);
  if (op == QMM_OP_MOE_SLOTS) return moe_workspace_bytes(M, K, T, E, top_k, false);
  if (op == QMM_OP_MOE_FFN) return moe_ffn_workspace_bytes(M, K, T, E, top_k);
  return 0;
}

extern "C" int qmm_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return QMM_ERR_NULL;
  if (!aligned16(ws)) return QMM_ERR_ALIGN;
  return zero_fill(ws, ws_bytes, to_stream(stream));
}

extern "C" int qmm_debug_subdots(int fmt, int path, const void* w, const void* xq, int32_t* D,
                                 int32_t* S, int64_t M, int64_t K, int64_t T, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (fmt != QMM_Q4_K && fmt != QMM_Q5_K && fmt != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  if (path != 0 && path != 1) return QMM_ERR_UNSUPPORTED;
  if (M < 1 || K < kQK || (K % kQK) != 0 || T < 1 || M > (1 << 20) || T > (1 << 20)) return QMM_ERR_SHAPE;
  if (path == 0 && T > QMM_MMVQ_MAX_T) return QMM_ERR_SHAPE;
  if (!w || !xq || !D || (fmt != QMM_Q6_K && !S)) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(D) || (S && !aligned16(S))) return QMM_ERR_ALIGN;
  if (path == 1 && (!ws || !aligned16(ws))) return ws ? QMM_ERR_ALIGN : QMM_ERR_NULL;
  if (path == 1 && ws_bytes < mmq_workspace_bytes(M, K, T)) return QMM_ERR_WORKSPACE;
  hipStream_t st = to_stream(stream);
  const int64_t nsub = fmt == QMM_Q6_K ? K / 16 : K / 32;
  int rc = zero_fill(D, static_cast<size_t>(T * M * nsub) * 4, st);
  if (rc == QMM_OK && fmt != QMM_Q6_K) rc = zero_fill(S, static_cast<size_t>(T * (K / 32)) * 4, st);
  if (rc != QMM_OK) return rc;
  if (path == 0) return debug_mmvq(fmt, w, xq, D, S, M, K, T, st);
  return mmq_dense(fmt, w, xq, nullptr, M, K, T, ws, st, D, S, nullptr);
}

extern "C" int qmm_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return QMM_ERR_NULL;
  if (!aligned16(buf) || !aligned16(sink)) return QMM_ERR_ALIGN;
  if (bytes == 0 || (bytes % 16) != 0) return QMM_ERR_SHAPE;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t grid = (n + 256 * kProbeUnroll - 1) / (256 * kProbeUnroll);
  if (grid > 0x7fffffff) return QMM_ERR_SHAPE;
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, to_stream(stream),
                     static_cast<const uint4*>(buf), n, sink);
  return launch_status();
}
