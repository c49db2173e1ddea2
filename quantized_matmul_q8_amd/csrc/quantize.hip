// Q8_1 activation quantizer and the SwiGLU -> Q8_1 glue.
//
// [8e] §2 fixes the rule (32-activation blocks, d = max|x|/127, round to the
// nearest integer, clamp to int8) and the "pad40" block (f16 d, two pad
// bytes, 32 int8 values on a 4-byte boundary, int32 sum for the min term);
// §3.2 shows the arithmetic (reciprocal multiply, round half to even).
// [MMQ] "What they do right": one byte per activation halves activation
// traffic.  The kernel is bound by HBM: it reads 4 bytes and writes 1.25
// bytes per activation.  Each group of eight lanes owns one 32-block, reads
// it as 8 x 16 bytes (one cache line per 8 lanes) and writes its 40 bytes.
#include "qmm_common.hpp"

namespace qmm {

__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float* __restrict__ x,
                                                            uint8_t* __restrict__ xq,
                                                            int64_t nblocks) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int part = static_cast<int>(gid & 7);
  const bool valid = blk < nblocks;
  const int64_t src = valid ? blk : 0;
  float4 v = reinterpret_cast<const float4*>(x)[src * 8 + part];
  if (!valid) v = make_float4(0.f, 0.f, 0.f, 0.f);
  // all lanes join the shuffles; only valid groups store
  q8_1_block_8lanes(v, part, xq + src * kQ8Bytes, valid);
}

// h = silu(g) * u for one 32-block of the output, then the Q8_1 quantizer.
// Row r of g_u holds gate in [0, F) and up in [F, 2F).
__global__ __launch_bounds__(256) void swiglu_q8_1_kernel(const float* __restrict__ g_u,
                                                          uint8_t* __restrict__ hq, int64_t R,
                                                          int64_t F) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t blk = gid >> 3;
  const int part = static_cast<int>(gid & 7);
  const int64_t bpr = F / kQB;  // blocks per row
  const bool valid = blk < R * bpr;
  const int64_t b = valid ? blk : 0;
  const int64_t r = b / bpr, c = (b % bpr) * kQB + part * 4;
  const float* row = g_u + r * 2 * F;
  const float4 g = *reinterpret_cast<const float4*>(row + c);
  const float4 u = *reinterpret_cast<const float4*>(row + F + c);
  float4 h;
  h.x = silu_mul(g.x, u.x);
  h.y = silu_mul(g.y, u.y);
  h.z = silu_mul(g.z, u.z);
  h.w = silu_mul(g.w, u.w);
  if (!valid) h = make_float4(0.f, 0.f, 0.f, 0.f);
  q8_1_block_8lanes(h, part, hq + b * kQ8Bytes, valid);
}

}  // namespace qmm

using namespace qmm;

extern "C" int q8_1_quantize(const float* x, void* xq, int64_t T, int64_t K, void* stream) {
  if (T < 0 || K <= 0 || (K % kQB) != 0) return QMM_ERR_SHAPE;
  if (T == 0) return QMM_OK;
  if (!x || !xq) return QMM_ERR_NULL;
  if (!aligned16(x) || !aligned16(xq)) return QMM_ERR_ALIGN;
  const int64_t nblocks = T * (K / kQB);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return QMM_ERR_SHAPE;
  hipLaunchKernelGGL(q8_1_quantize_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     to_stream(stream), x, static_cast<uint8_t*>(xq), nblocks);
  return launch_status();
}

extern "C" int swiglu_q8_1(const float* g_u, void* hq, int64_t R, int64_t F, void* stream) {
  if (R < 0 || F <= 0 || (F % kQB) != 0) return QMM_ERR_SHAPE;
  if (R == 0) return QMM_OK;
  if (!g_u || !hq) return QMM_ERR_NULL;
  if (!aligned16(g_u) || !aligned16(hq)) return QMM_ERR_ALIGN;
  const int64_t threads = R * (F / kQB) * 8;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7fffffff) return QMM_ERR_SHAPE;
  hipLaunchKernelGGL(swiglu_q8_1_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     to_stream(stream), g_u, static_cast<uint8_t*>(hq), R, F);
  return launch_status();
}
