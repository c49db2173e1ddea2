// Measurement hooks, not part of the method: ceilings that the GEMM's and the
// matvec's measured rates are read against.
//
// * qmm_probe_mfma: back-to-back int8 MFMA (v_mfma_i32_32x32x32_i8) from
//   registers, four independent accumulators per wave -- the matrix-core
//   rate the int8 peak assumes.
// * qmm_probe_mfma_epilogue: the GEMM's per-sub-block inner loop without
//   global memory: one int8 MFMA per 32 x 32 output block started from the
//   bits of 1.5*2^23, then the two fp32 FMAs per output element that turn the
//   integer sums into the scaled fp32 accumulation (beta*D rounded once, then
//   alpha*that added), software pipelined over two column blocks as the
//   kernel is; optionally with the operands read from LDS as the kernel reads
//   them and with the Q4_K min-term fp32 MFMA every second sub-block.  This
//   is the "per-subblock rescale epilogue tax" of [GAP] root cause 1 measured
//   on its own; [MMQ] "Revised priorities (post-M3 findings)" asks for the
//   dequant/epilogue ALU cost to be measured before tuning around it.
// * qmm_probe_read_geom: the read-only HBM probe of qmm_probe_read with its
//   geometry as arguments (16-byte loads in flight per thread, grid size or
//   a persistent grid-stride loop), for sweeping the read ceiling ([8e] §6:
//   measure a read-only ceiling, concurrency first).
// Every loop has a trip count fixed by its arguments and every access stays
// inside the caller's buffer or the kernel's own LDS array.
#include "qmm_common.hpp"

namespace qmm {

constexpr int kProbeThreads = 512;  // eight waves: two per SIMD per workgroup
constexpr uint32_t kProbeMagicBits = 0x4B400000u;
constexpr float kProbeMagic = 12582912.0f;

__device__ __forceinline__ void opaque(v4i& v) { __asm__ volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(v16i& v) { __asm__ volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(float& v) { __asm__ volatile("" : "+v"(v)); }

__device__ __forceinline__ void probe_sink(uint32_t acc, uint32_t* sink) {
  if (acc == 0x9e3779b9u) sink[0] = acc;  // practically never: keeps the work live
}

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int64_t iters, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  v4i a = {lane, lane * 3, lane * 5, lane * 7};
  v4i b = {lane * 11, lane * 13, lane * 17, lane * 19};
  opaque(a);
  opaque(b);
  v16i c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) c[j][v] = j;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc ^= static_cast<uint32_t>(c[j][v]);
  probe_sink(acc, sink);
}

// MODE 1: operands in registers; 2: alpha, beta and the B operand read from
// LDS each sub-block (the kernel's reads: 16 row scales per lane, a (beta,
// -beta*C) pair and 16 B bytes per column block); 3: as 2 plus the min-term
// fp32 MFMA every second sub-block into the epilogue's accumulator; 4: the
// same MFMA into an accumulator of its own (no dependency between the FMA
// chain and the matrix core); 5: as 4 with the min term as three bf16 MFMAs
// per super-block (K = 16 each: a three-way bf16 split of -dmin*m against one
// of beta*S, six of the nine partial products); 6: as 5 into the epilogue's
// accumulator; 7: as 6 with a workgroup barrier every eight sub-blocks (the
// GEMM's step); 8: as 7 with the A operand unpacked from 4-bit values each
// sub-block.  Two column blocks (NT = 2).
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void probe_epilogue_kernel(int64_t iters, uint32_t* sink) {
  constexpr int NT = 2;
  __shared__ __attribute__((aligned(16))) float s_al[8][32];      // alpha[sub-block][row]
  __shared__ __attribute__((aligned(16))) float2 s_bp[8][NT][32]; // (beta, -beta*C)[sub-block][ct][col]
  __shared__ __attribute__((aligned(16))) v4i s_bq[8][NT][64];    // B operand[sub-block][ct][lane]
  __shared__ __attribute__((aligned(16))) float s_bm[8][NT][64];  // min-term B[sub-block][ct][lane]
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  for (int i = threadIdx.x; i < 8 * 32; i += kProbeThreads) (&s_al[0][0])[i] = 1.0f + 1e-3f * (i & 15);
  for (int i = threadIdx.x; i < 8 * NT * 32; i += kProbeThreads)
    (&s_bp[0][0][0])[i] = make_float2(0.5f, -0.5f * kProbeMagic);
  for (int i = threadIdx.x; i < 8 * NT * 64; i += kProbeThreads) {
    (&s_bq[0][0][0])[i] = v4i{i, 3 * i, 5 * i, 7 * i};
    (&s_bm[0][0][0])[i] = 1e-3f;
  }
  __syncthreads();
  v4i a = {lane, lane * 3, lane * 5, lane * 7};
  opaque(a);
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = static_cast<int>(kProbeMagicBits);
  opaque(magic);
  float al_r[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    al_r[v] = 1.0f + 1e-3f * v;
    opaque(al_r[v]);
  }
  float2 bp_r[NT];
  v4i bq_r[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    bp_r[ct] = make_float2(0.5f, -0.5f * kProbeMagic);
    opaque(bp_r[ct].x);
    opaque(bp_r[ct].y);
    bq_r[ct] = v4i{lane * (ct + 11), lane * 13, lane * 17, lane * 19};
    opaque(bq_r[ct]);
  }
  float am = 1e-3f;
  opaque(am);
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  v8bf abf, bbf[NT];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    abf[k] = static_cast<__bf16>(1.0f + k);
    bbf[0][k] = static_cast<__bf16>(0.5f * k);
    bbf[1][k] = static_cast<__bf16>(0.25f * k);
  }
  __asm__ volatile("" : "+v"(abf));
  v16f acc[NT], accm[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    __asm__ volatile("" : "+v"(bbf[ct]));
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ct][v] = accm[ct][v] = 0.0f;
  }
  v16i X[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) X[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq_r[ct], magic, 0, 0, 0);
  for (int64_t i = 0; i < iters; ++i) {
    const int u = static_cast<int>(i & 7);
    float al[16];
    float2 bp[NT];
    v4i bq[NT];
    float bm[NT];
    if constexpr (MODE >= 2) {
      const float* wa = &s_al[u][4 * g];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 t4 = *reinterpret_cast<const float4*>(wa + 8 * k);
        al[4 * k] = t4.x; al[4 * k + 1] = t4.y; al[4 * k + 2] = t4.z; al[4 * k + 3] = t4.w;
      }
      const int un = (u + 1) & 7;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        bp[ct] = s_bp[u][ct][col];
        bq[ct] = s_bq[un][ct][lane];   // the next sub-block's B operand
        bm[ct] = s_bm[u][ct][lane];
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) al[v] = al_r[v];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        bp[ct] = bp_r[ct];
        bq[ct] = bq_r[ct];
        opaque(bq[ct]);
        bm[ct] = am;
      }
    }
    if constexpr (MODE >= 8) {
      // the A operand unpacked from 4-bit values as the GEMM does
      const int sh = (u & 1) * 4;
      a = v4i{static_cast<int>((static_cast<uint32_t>(a[0]) >> sh) & 0x0f0f0f0fu),
              static_cast<int>((static_cast<uint32_t>(a[1]) >> sh) & 0x0f0f0f0fu),
              static_cast<int>((static_cast<uint32_t>(a[2]) >> sh) & 0x0f0f0f0fu),
              static_cast<int>((static_cast<uint32_t>(a[3]) >> sh) & 0x0f0f0f0fu)};
    }
    opaque(a);
    if constexpr (MODE >= 7) {
      if (u == 7) __syncthreads();   // one barrier per eight sub-blocks, as the GEMM's step
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const v16f Xf = __builtin_bit_cast(v16f, X[ct]);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float t = __builtin_fmaf(bp[ct].x, Xf[v], bp[ct].y);
        acc[ct][v] = __builtin_fmaf(al[v], t, acc[ct][v]);
      }
      if constexpr (MODE == 3) {
        if (u & 1) acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(am, bm[ct], acc[ct], 0, 0, 0);
      } else if constexpr (MODE == 4) {
        if (u & 1) accm[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(am, bm[ct], accm[ct], 0, 0, 0);
      } else if constexpr (MODE >= 5) {
        // once per super-block (8 sub-blocks): three bf16 MFMAs (K = 3 x 16),
        // spread over the sub-blocks; into an accumulator of its own (5) or
        // into the epilogue's (6)
        if (u == 1 || u == 3 || u == 5) {
          if constexpr (MODE == 5)
            accm[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abf, bbf[ct], accm[ct], 0, 0, 0);
          else if constexpr (MODE >= 7)
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abf, bbf[ct], acc[ct], 0, 0, 0);
          else
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abf, bbf[ct], acc[ct], 0, 0, 0);
        }
      }
      X[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq[ct], magic, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the accumulators and the last MFMA results are folded into the sink test
  // (a float sum for the accumulators: an xor of them may cancel symbolically)
  float fs = 0.0f;
  uint32_t h = 0;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      fs += (acc[ct][v] + accm[ct][v]) * static_cast<float>(1 + v + 16 * ct);
      h ^= static_cast<uint32_t>(X[ct][v]);
    }
  probe_sink(h ^ __builtin_bit_cast(uint32_t, fs), sink);
}

// The one-column-block inner loop (the grouped-expert GEMM's): per sub-block
// its B operand and column factors read from LDS, the int8 MFMA, then the
// epilogue with the row scales read from LDS four at a time, no software
// pipelining; three bf16 min-term MFMAs and one workgroup barrier per eight
// sub-blocks.  Runs at four waves per SIMD (two workgroups per CU).
__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void probe_lean_kernel(int64_t iters, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) float s_al[8][32];
  __shared__ __attribute__((aligned(16))) float2 s_bp[8][32];
  __shared__ __attribute__((aligned(16))) v4i s_bq[8][64];
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  for (int i = threadIdx.x; i < 8 * 32; i += kProbeThreads) {
    (&s_al[0][0])[i] = 1.0f + 1e-3f * (i & 15);
    (&s_bp[0][0])[i] = make_float2(0.5f, -0.5f * kProbeMagic);
  }
  for (int i = threadIdx.x; i < 8 * 64; i += kProbeThreads) (&s_bq[0][0])[i] = v4i{i, 3 * i, 5 * i, 7 * i};
  __syncthreads();
  v4i a = {lane, lane * 3, lane * 5, lane * 7};
  opaque(a);
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = static_cast<int>(kProbeMagicBits);
  opaque(magic);
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  v8bf abf, bbf;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    abf[k] = static_cast<__bf16>(1.0f + k);
    bbf[k] = static_cast<__bf16>(0.5f * k);
  }
  __asm__ volatile("" : "+v"(abf), "+v"(bbf));
  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  for (int64_t i = 0; i < iters; ++i) {
    const int u = static_cast<int>(i & 7);
    const v4i bq = s_bq[u][lane];
    const float2 bp = s_bp[u][col];
    opaque(a);
    const v16i X = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, magic, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    const v16f Xf = __builtin_bit_cast(v16f, X);
    const float* wa = &s_al[u][4 * g];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a4 = *reinterpret_cast<const float4*>(wa + 8 * k);
      const float al4[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[4 * k + j] = __builtin_fmaf(al4[j], __builtin_fmaf(bp.x, Xf[4 * k + j], bp.y),
                                                                   acc[4 * k + j]);
    }
    if (u == 1 || u == 3 || u == 5) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abf, bbf, acc, 0, 0, 0);
    if (u == 7) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  float fs = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) fs += acc[v] * static_cast<float>(1 + v);
  probe_sink(__builtin_bit_cast(uint32_t, fs), sink);
}

// Read-only streaming with a chosen geometry.  U 16-byte loads per thread
// are issued before any is used (U in flight), lane-contiguous, one grid
// stride apart; the grid then strides over the buffer until every chunk of
// U * grid * 256 loads is read (a one-pass grid has a single round).
template <int U>
__global__ __launch_bounds__(256) void probe_read_geom_kernel(const uint4* __restrict__ p, int64_t n,
                                                              uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; base < n; base += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * stride;
      v[u] = i < n ? ld16_nt(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  probe_sink(acc, sink);
}

static int probe_grid(int waves_per_simd) {
  // eight waves (two per SIMD) per workgroup
  return device_cu_count() * (waves_per_simd / 2);
}

}  // namespace qmm

using namespace qmm;

extern "C" int qmm_probe_mfma(int64_t iters, int waves_per_simd, uint32_t* sink, void* stream) {
  if (!sink) return QMM_ERR_NULL;
  if (!aligned16(sink)) return QMM_ERR_ALIGN;
  if (iters < 1 || iters > (int64_t{1} << 24)) return QMM_ERR_SHAPE;
  if (waves_per_simd != 2 && waves_per_simd != 4 && waves_per_simd != 8) return QMM_ERR_SHAPE;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(probe_grid(waves_per_simd)), dim3(kProbeThreads), 0, to_stream(stream),
                     iters, sink);
  return launch_status();
}

extern "C" int qmm_probe_mfma_epilogue(int mode, int64_t iters, int waves_per_simd, uint32_t* sink, void* stream) {
  if (!sink) return QMM_ERR_NULL;
  if (!aligned16(sink)) return QMM_ERR_ALIGN;
  if (mode < 1 || mode > 9) return QMM_ERR_UNSUPPORTED;
  if (iters < 1 || iters > (int64_t{1} << 24)) return QMM_ERR_SHAPE;
  if (waves_per_simd != 2 && waves_per_simd != 4) return QMM_ERR_SHAPE;
  const dim3 grid(probe_grid(waves_per_simd)), block(kProbeThreads);
  hipStream_t st = to_stream(stream);
  if (mode == 1) hipLaunchKernelGGL(probe_epilogue_kernel<1>, grid, block, 0, st, iters, sink);
  if (mode == 2) hipLaunchKernelGGL(probe_epilogue_kernel<2>, grid, block, 0, st, iters, sink);
  if (mode == 3) hipLaunchKernelGGL(probe_epilogue_kernel<3>, grid, block, 0, st, iters, sink);
  if (mode == 4) hipLaunchKernelGGL(probe_epilogue_kernel<4>, grid, block, 0, st, iters, sink);
  if (mode == 5) hipLaunchKernelGGL(probe_epilogue_kernel<5>, grid, block, 0, st, iters, sink);
  if (mode == 6) hipLaunchKernelGGL(probe_epilogue_kernel<6>, grid, block, 0, st, iters, sink);
  if (mode == 7) hipLaunchKernelGGL(probe_epilogue_kernel<7>, grid, block, 0, st, iters, sink);
  if (mode == 8) hipLaunchKernelGGL(probe_epilogue_kernel<8>, grid, block, 0, st, iters, sink);
  // mode 9: the one-column-block loop, ops per launch counted as one MFMA per
  // iteration (half those of modes 1-8), always two workgroups per CU
  if (mode == 9) hipLaunchKernelGGL(probe_lean_kernel, dim3(device_cu_count() * 2), block, 0, st, iters, sink);
  return launch_status();
}

extern "C" int qmm_probe_read_geom(const void* buf, size_t bytes, int loads_per_thread, int64_t grid,
                                   uint32_t* sink, void* stream) {
  if (!buf || !sink) return QMM_ERR_NULL;
  if (!aligned16(buf) || !aligned16(sink)) return QMM_ERR_ALIGN;
  if (bytes == 0 || (bytes % 16) != 0) return QMM_ERR_SHAPE;
  const int U = loads_per_thread;
  if (U != 1 && U != 2 && U != 4 && U != 8 && U != 16) return QMM_ERR_SHAPE;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t one_pass = (n + 256 * U - 1) / (256 * U);
  if (grid <= 0 || grid > one_pass) grid = one_pass;  // 0: one pass, U loads per thread
  if (grid > 0x7fffffff) return QMM_ERR_SHAPE;
  const dim3 g(static_cast<unsigned>(grid)), b(256);
  hipStream_t st = to_stream(stream);
  const uint4* p = static_cast<const uint4*>(buf);
  switch (U) {
    case 1: hipLaunchKernelGGL(probe_read_geom_kernel<1>, g, b, 0, st, p, n, sink); break;
    case 2: hipLaunchKernelGGL(probe_read_geom_kernel<2>, g, b, 0, st, p, n, sink); break;
    case 4: hipLaunchKernelGGL(probe_read_geom_kernel<4>, g, b, 0, st, p, n, sink); break;
    case 8: hipLaunchKernelGGL(probe_read_geom_kernel<8>, g, b, 0, st, p, n, sink); break;
    default: hipLaunchKernelGGL(probe_read_geom_kernel<16>, g, b, 0, st, p, n, sink); break;
  }
  return launch_status();
}
