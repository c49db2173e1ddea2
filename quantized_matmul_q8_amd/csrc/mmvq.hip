// Decode matvec (MMVQ): y[t][i] = sum_k W[i][k] * x_t[k] for T <= 8 tokens,
// Q4_K or Q6_K weights against Q8_1 activations.
//
// Method ([8e] §2 and §3.2): weights stay packed in HBM and are unpacked in
// registers to small integers; each 4-weight group is multiplied with four
// int8 activations by one integer dot instruction.  For Q4_K the min term of
// every 32-weight sub-block needs the sub-block's activation sum, obtained by
// a dot product of the int8 activations with 0x01010101:
//   W.x = sum_s dx_s * ( d*sc_s * sum(nib*q) - dmin*m_s * sum(q) ).
// Q6_K uses the signed values q6 - 32, so no min term is needed; its dot is
// sum(q6*q) - 32*sum(q), again with the ones dot.
//
// Geometry (re-derived for MI355X; [8e] §2 "the MMVQ geometry" is the
// 256-thread-per-row prior art for a 48-SM LPDDR part): one wave64 per weight
// row, four rows per 256-thread workgroup.  The row's (super-block, part)
// units are dealt round-robin to the 64 lanes; a Q4_K unit is 16 bytes of
// packed values (32 weights: 16 of sub-block 2p, 16 of 2p+1), so consecutive
// lanes read consecutive 16-byte chunks of a block and every dwordx4 load of
// the wave covers ~1 KB of the row.  At M = 4096 the grid holds 4096 waves
// (16 per CU), enough loads in flight to cover HBM latency.  The row sum is a
// wave reduction; lane 0 writes y[t*M + row].  Loads of weights are
// non-temporal: each byte is used once and must not evict the activations.
#include "qmm_common.hpp"

namespace qmm {

constexpr int kMmvqRowsPerBlock = 4;

// DEBUG == true: write the integer sub-block sums (D per (t, row, sub-block),
// S per (t, sub-block) from row 0) with integer atomics into zeroed buffers,
// instead of the scaled result.  Same loads, unpacking and dot products.
template <int T, bool DEBUG>
__global__ __launch_bounds__(256) void mmvq_q4k_kernel(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ xq,
                                                       float* __restrict__ y, int M, int nb,
                                                       int32_t* __restrict__ dbgD,
                                                       int32_t* __restrict__ dbgS) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMmvqRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wave
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * kQ4Bytes;
  const int nunits = nb * 8;
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  for (int u = lane; u < nunits; u += 64) {
    const int b = u >> 3, c = u & 7, p = c >> 1, h = c & 1;
    const uint8_t* blk = wrow + b * kQ4Bytes;
    const uint4 hdr = ld16_nt(blk);
    const uint4 qv = ld16_nt(blk + 16 + 32 * p + 16 * h);
    int sc0, m0, sc1, m1;
    q4k_scale_min(2 * p, hdr.y, hdr.z, hdr.w, sc0, m0);
    q4k_scale_min(2 * p + 1, hdr.y, hdr.z, hdr.w, sc1, m1);
    const float d = h2f(hdr.x & 0xffffu), dmin = h2f(hdr.x >> 16);
    const float ds0 = d * static_cast<float>(sc0), dm0 = dmin * static_cast<float>(m0);
    const float ds1 = d * static_cast<float>(sc1), dm1 = dmin * static_cast<float>(m1);
    const uint32_t lo0 = qv.x & 0x0f0f0f0fu, lo1 = qv.y & 0x0f0f0f0fu;
    const uint32_t lo2 = qv.z & 0x0f0f0f0fu, lo3 = qv.w & 0x0f0f0f0fu;
    const uint32_t hi0 = (qv.x >> 4) & 0x0f0f0f0fu, hi1 = (qv.y >> 4) & 0x0f0f0f0fu;
    const uint32_t hi2 = (qv.z >> 4) & 0x0f0f0f0fu, hi3 = (qv.w >> 4) & 0x0f0f0f0fu;
    const int sb0 = b * 8 + 2 * p;  // Q8_1 block of sub-block 2p (2p+1 follows)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint8_t* xb = xq + t * xstride + static_cast<size_t>(sb0) * kQ8Bytes;
      const uint4 x0 = ld16_a4(xb + 4 + 16 * h);
      const uint4 x1 = ld16_a4(xb + kQ8Bytes + 4 + 16 * h);
      const float dx0 = h2f(ld_u16(xb)), dx1 = h2f(ld_u16(xb + kQ8Bytes));
      int D0 = dot4(lo0, x0.x, 0);
      D0 = dot4(lo1, x0.y, D0);
      D0 = dot4(lo2, x0.z, D0);
      D0 = dot4(lo3, x0.w, D0);
      int S0 = dot4(0x01010101u, x0.x, 0);
      S0 = dot4(0x01010101u, x0.y, S0);
      S0 = dot4(0x01010101u, x0.z, S0);
      S0 = dot4(0x01010101u, x0.w, S0);
      int D1 = dot4(hi0, x1.x, 0);
      D1 = dot4(hi1, x1.y, D1);
      D1 = dot4(hi2, x1.z, D1);
      D1 = dot4(hi3, x1.w, D1);
      int S1 = dot4(0x01010101u, x1.x, 0);
      S1 = dot4(0x01010101u, x1.y, S1);
      S1 = dot4(0x01010101u, x1.z, S1);
      S1 = dot4(0x01010101u, x1.w, S1);
      if constexpr (DEBUG) {
        int32_t* Dt = dbgD + (static_cast<size_t>(t) * M + row) * (nb * 8);
        atomicAdd(Dt + sb0, D0);
        atomicAdd(Dt + sb0 + 1, D1);
        if (row == 0) {
          atomicAdd(dbgS + static_cast<size_t>(t) * nb * 8 + sb0, S0);
          atomicAdd(dbgS + static_cast<size_t>(t) * nb * 8 + sb0 + 1, S1);
        }
      } else {
        acc[t] += dx0 * (ds0 * static_cast<float>(D0) - dm0 * static_cast<float>(S0)) +
                  dx1 * (ds1 * static_cast<float>(D1) - dm1 * static_cast<float>(S1));
      }
    }
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

// Q6_K unit: one half h of the super-block and 16 lanes l0..l0+15 of it, i.e.
// 64 weights in four 16-weight sub-blocks (g = 0..3 at positions
// 128h + 32g + l).  Bytes used: ql[64h + l0 ..+16], ql[64h + 32 + l0 ..+16],
// qh[32h + l0 ..+16], four scales and d.  Blocks are 2-byte aligned.
template <int T, bool DEBUG>
__global__ __launch_bounds__(256) void mmvq_q6k_kernel(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ xq,
                                                       float* __restrict__ y, int M, int nb,
                                                       int32_t* __restrict__ dbgD) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMmvqRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * kQ6Bytes;
  const int nunits = nb * 4;
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  for (int u = lane; u < nunits; u += 64) {
    const int b = u >> 2, c = u & 3, h = c >> 1, half16 = c & 1, l0 = half16 * 16;
    const uint8_t* blk = wrow + static_cast<size_t>(b) * kQ6Bytes;
    const uint4 qa = ld16_a2(blk + 64 * h + l0);        // g = 0 (low nibbles), g = 2 (high)
    const uint4 qb = ld16_a2(blk + 64 * h + 32 + l0);   // g = 1 (low nibbles), g = 3 (high)
    const uint4 qh = ld16_a2(blk + 128 + 32 * h + l0);  // bit pairs of g = 0..3
    const float d = h2f(ld_u16(blk + 208));
    float dsc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t two = ld_u16(blk + 192 + 8 * h + 2 * g);  // sc[8h+2g], sc[8h+2g+1]
      const int sc = static_cast<int8_t>((two >> (8 * half16)) & 0xffu);
      dsc[g] = d * static_cast<float>(sc);
    }
    const uint32_t qa_[4] = {qa.x, qa.y, qa.z, qa.w};
    const uint32_t qb_[4] = {qb.x, qb.y, qb.z, qb.w};
    const uint32_t qh_[4] = {qh.x, qh.y, qh.z, qh.w};
    uint32_t q6[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q6[0][k] = (qa_[k] & 0x0f0f0f0fu) | ((qh_[k] << 4) & 0x30303030u);
      q6[1][k] = (qb_[k] & 0x0f0f0f0fu) | ((qh_[k] << 2) & 0x30303030u);
      q6[2][k] = ((qa_[k] >> 4) & 0x0f0f0f0fu) | (qh_[k] & 0x30303030u);
      q6[3][k] = ((qb_[k] >> 4) & 0x0f0f0f0fu) | ((qh_[k] >> 2) & 0x30303030u);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int sblk = b * 8 + 4 * h + g;  // Q8_1 block holding these weights
        const uint8_t* xb = xq + t * xstride + static_cast<size_t>(sblk) * kQ8Bytes;
        const uint4 xv = ld16_a4(xb + 4 + l0);
        const float dx = h2f(ld_u16(xb));
        int D = dot4(q6[g][0], xv.x, 0);
        D = dot4(q6[g][1], xv.y, D);
        D = dot4(q6[g][2], xv.z, D);
        D = dot4(q6[g][3], xv.w, D);
        int S = dot4(0x01010101u, xv.x, 0);
        S = dot4(0x01010101u, xv.y, S);
        S = dot4(0x01010101u, xv.z, S);
        S = dot4(0x01010101u, xv.w, S);
        const int D6 = D - 32 * S;  // sum (q6 - 32) * q, exact
        if constexpr (DEBUG) {
          dbgD[(static_cast<size_t>(t) * M + row) * (nb * 16) + sblk * 2 + half16] = D6;
        } else {
          acc[t] += dx * dsc[g] * static_cast<float>(D6);
        }
      }
    }
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

template <bool DEBUG>
static int launch_mmvq_q4k(const void* w, const void* xq, float* y, int M, int nb, int T,
                           int32_t* D, int32_t* S, hipStream_t st) {
  const dim3 grid((M + kMmvqRowsPerBlock - 1) / kMmvqRowsPerBlock), block(256);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint8_t* xp = static_cast<const uint8_t*>(xq);
  switch (T) {
#define QMM_CASE(TT) \
  case TT: hipLaunchKernelGGL((mmvq_q4k_kernel<TT, DEBUG>), grid, block, 0, st, wp, xp, y, M, nb, D, S); break;
    QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
    default: return QMM_ERR_SHAPE;
  }
  return launch_status();
}

template <bool DEBUG>
static int launch_mmvq_q6k(const void* w, const void* xq, float* y, int M, int nb, int T,
                           int32_t* D, hipStream_t st) {
  const dim3 grid((M + kMmvqRowsPerBlock - 1) / kMmvqRowsPerBlock), block(256);
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint8_t* xp = static_cast<const uint8_t*>(xq);
  switch (T) {
#define QMM_CASE(TT) \
  case TT: hipLaunchKernelGGL((mmvq_q6k_kernel<TT, DEBUG>), grid, block, 0, st, wp, xp, y, M, nb, D); break;
    QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
    default: return QMM_ERR_SHAPE;
  }
  return launch_status();
}

// Host checks shared by both formats.
static int check_mmvq(const void* w, const void* xq, const float* y, int64_t M, int64_t K, int64_t T) {
  if (M < 1 || K < kQK || (K % kQK) != 0 || T < 1 || T > QMM_MMVQ_MAX_T) return QMM_ERR_SHAPE;
  if (M > 0x7fffffff || K / kQK > (1 << 20)) return QMM_ERR_SHAPE;
  if (!w || !xq || !y) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(y)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

int debug_mmvq(int fmt, const void* w, const void* xq, int32_t* D, int32_t* S, int64_t M,
               int64_t K, int64_t T, hipStream_t st) {
  if (fmt == QMM_Q4_K)
    return launch_mmvq_q4k<true>(w, xq, nullptr, static_cast<int>(M), static_cast<int>(K / kQK),
                                 static_cast<int>(T), D, S, st);
  return launch_mmvq_q6k<true>(w, xq, nullptr, static_cast<int>(M), static_cast<int>(K / kQK),
                               static_cast<int>(T), D, st);
}

}  // namespace qmm

using namespace qmm;

extern "C" int mmvq_q4k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                        void* stream) {
  const int st = check_mmvq(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  return launch_mmvq_q4k<false>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK),
                                static_cast<int>(T), nullptr, nullptr, to_stream(stream));
}

extern "C" int mmvq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                        void* stream) {
  const int st = check_mmvq(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  return launch_mmvq_q6k<false>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK),
                                static_cast<int>(T), nullptr, to_stream(stream));
}
