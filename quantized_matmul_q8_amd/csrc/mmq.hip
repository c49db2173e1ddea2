// Prefill GEMM (MMQ) and its MoE grouped form: y[t][i] = sum_k W[i][k] x_t[k]
// for many tokens, Q4_K or Q6_K weights against Q8_1 activations, on int8
// MFMA with int32 accumulation per sub-block and an fp32 epilogue.
//
// Prior art: [MMQ] "Kernel architecture" (128x128 tiles of weights x tokens,
// dequant fused into the matrix inner loop, Q8_1 activations, persistent
// workgroups claiming tiles from an atomic counter instead of Stream-K plus a
// fixup pass, MoE work entries (expert, m_tile, n_tile)); [GAP] root cause 1
// and lever T1; [8e] §2 for the min-term factorisation.  Re-designed for
// gfx950 as follows.
//
// * Matrix core.  One v_mfma_i32_32x32x32_i8 covers exactly one 32-weight
//   Q4_K sub-block of 32 rows x 32 tokens: A = unpacked 4-bit values (0..15),
//   B = the Q8_1 int8 values, int32 result D per (row, token, sub-block).  Q6_K
//   has 16-weight sub-blocks and uses v_mfma_i32_32x32x16_i8 per sub-block,
//   with the unsigned 6-bit values as A.
// * Epilogue.  Every (row i, token j, sub-block s) has its own factor
//   alpha_is * beta_js (weight scale d*sc, activation scale d_x), so each
//   MFMA result is rescaled before the next sub-block.  The MFMA accumulator
//   starts at the bit pattern of 1.5*2^23; since |D| < 2^22 the int32 result
//   read as fp32 is exactly 1.5*2^23 + D.  Then
//     t   = fma(beta, X, -beta*1.5*2^23)   = beta*D, rounded once
//     acc = fma(alpha, t, acc)
//   i.e. two fp32 VALU ops per output element per sub-block, no conversion.
// * Min term.  sum_s (-dmin*m_is) * (beta_js*S_js) is a small GEMM over the
//   sub-block index; it runs on v_mfma_f32_32x32x2_f32 straight into the fp32
//   accumulator (Q6_K: the -32 offset of the signed values, the same way).
// * Work queue.  Persistent grid; tiles are split into 8 contiguous ranges,
//   one per XCD (workgroup b runs on XCD b % 8), each with its own atomic
//   counter, so the weight rows of a range stay in one XCD's L2.  A workgroup
//   that drains its range helps the others.  Tiles run their whole K loop in
//   one workgroup: no split-K, no fixup, deterministic results.  The last
//   workgroup to leave resets the counters, so the workspace is zero again
//   for the next call without a memset.
#include "qmm_common.hpp"

#include <type_traits>

namespace qmm {

constexpr int kMmqThreads = 256;       // 4 waves
constexpr int kMmqBM = 128;            // weight rows per tile (32 per wave)
constexpr uint32_t kMagicBits = 0x4B400000u;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

enum MmqMode { kDense = 0, kMoe = 1, kDebug = 2 };

struct MmqParams {
  const uint8_t* w;
  const uint8_t* xq;
  float* y;
  int M, nb, T;                 // rows, super-blocks per row, tokens (dense)
  unsigned* counters;           // kXcds queue counters, then the exit counter
  // MoE (mode kMoe)
  const int32_t* counts;        // [E] routed slots per expert
  const int32_t* offsets;       // [E+1] slot offsets into bucket
  const int32_t* bucket;        // [T*top_k] slots grouped by expert
  const int32_t* work_off;      // [E+1] prefix of (m_tiles * n_tiles(e))
  int E, top_k, rows_per_token;
  int64_t expert_stride;
  // debug (mode kDebug)
  int32_t* dbgD;
  int32_t* dbgS;
};

// LDS of one pipeline stage (two stages are used, double-buffered).
// Activation payload: for each Q8_1 block s of the super-block, the 32 int8
// values of every column are cut into pieces (Q4_K 2 x 16 bytes: one MFMA
// k-group each; Q6_K 4 x 8 bytes) and piece k of all columns is one
// contiguous run, so the MFMA operand reads of 32 consecutive columns are
// consecutive.  Rows of s are padded by 32 bytes so that the commit stores
// (8 lanes = the 8 blocks of one token, next 8 lanes = next token) of any
// 16 lanes (16-byte pieces) or 32 lanes (8-byte pieces) fall on distinct
// banks; reads stay a per-lane base plus immediate offsets.
template <int FMT, int NT>
struct MmqSmem {
  static constexpr int BN = 32 * NT;
  static constexpr int NS16 = FMT == QMM_Q4_K ? 8 : 16;     // scale groups per super-block
  static constexpr int kPiece = FMT == QMM_Q4_K ? 16 : 8;    // payload bytes per piece
  static constexpr int kXqRow = 32 * BN + 32;               // bytes per block row s
  static constexpr int kXbRow = BN + 4;                      // float2 per block row
  static constexpr int kXsRow = BN + 8;                      // floats per beta*S row
  static constexpr int kXq = 0;                              // [8][32/kPiece][BN][kPiece] int8 payload
  static constexpr int kXb = kXq + 8 * kXqRow;               // [8][kXbRow] (beta, -beta*C)
  static constexpr int kXs = kXb + 8 * kXbRow * 8;           // Q4_K: [8][kXsRow] beta*S
  static constexpr int kWa = kXs + (FMT == QMM_Q4_K ? 8 * kXsRow * 4 : 0);  // [4 waves][NS16][32] alpha = d*sc
  static constexpr int kWm = kWa + 4 * NS16 * 32 * 4;        // Q4_K: [4][8][32] -dmin*m
  static constexpr int kStage = (kWm + (FMT == QMM_Q4_K ? 4 * 8 * 32 * 4 : 0) + 15) & ~15;
  static constexpr int kBytes = 2 * kStage;
};

// Token (activation row, output row) of column j of a tile.  Dense: token
// n0 + j (clamped for loads).  MoE: the j-th routed slot of the tile.
struct TileCols {
  int n0, ncols;      // first column, valid columns
  int slot_base;      // MoE: offset of the expert's slots in bucket
};

template <int MODE>
__device__ __forceinline__ void col_rows(const MmqParams& P, const TileCols& tc, int j, int& xrow,
                                         int& orow, bool& valid) {
  const int jj = min(j, tc.ncols - 1);
  valid = j < tc.ncols;
  if constexpr (MODE == kMoe) {
    const int slot = P.bucket[tc.slot_base + tc.n0 + jj];
    xrow = P.rows_per_token == 1 ? slot / P.top_k : slot;
    orow = slot;
  } else {
    xrow = tc.n0 + jj;
    orow = xrow;
  }
}

// Registers holding one super-block's global data between its loads and
// its commit to LDS (the software pipeline's in-flight stage).
template <int FMT, int NT>
struct MmqPrefetch {
  static constexpr int RX = 32 * NT * 8 / kMmqThreads;  // Q8_1 blocks staged per thread
  uint2 xu[RX][5];                                      // raw 40-byte activation blocks
  // Q4_K: header and the 4 x 16 value bytes of this lane's row and k-group
  uint4 hdr;
  uint4 q[4];
  // Q6_K: per (half h, 16-group hf): qh bytes; per (h, parity, hf): ql bytes
  // (8 bytes each as raw aligned dwords + shift), scales of this k-group, d
  uint32_t qh_raw[2][2][3], ql_raw[2][2][2][3], sc_raw[3], d_raw, sh;
};

// 8 bytes at p (2-byte aligned) from three raw aligned dwords and the shift.
__device__ __forceinline__ void raw8_load(const uint8_t* p, uint32_t (&r)[3], uint32_t& sh) {
  sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p - sh);  // stays a global pointer
  r[0] = base[0];
  r[1] = base[1];
  r[2] = sh ? base[2] : 0u;  // only when misaligned: never reads past p + 8 otherwise
}
__device__ __forceinline__ uint2 raw8_join(const uint32_t (&r)[3], uint32_t sh) {
  return make_uint2(__builtin_amdgcn_alignbyte(r[1], r[0], sh), __builtin_amdgcn_alignbyte(r[2], r[1], sh));
}

// Issue the global loads of super-block sb (activations of the tile's
// columns, this lane's weight bytes) into registers.
template <int FMT, int NT>
__device__ __forceinline__ void mmq_load(const MmqParams& P, MmqPrefetch<FMT, NT>& F, const int* xrow,
                                         size_t xstride, const uint8_t* wr, int sb, int g) {
#pragma unroll
  for (int r = 0; r < MmqPrefetch<FMT, NT>::RX; ++r) {
    const int s = (threadIdx.x + kMmqThreads * r) & 7;
    const uint2* src = reinterpret_cast<const uint2*>(P.xq + static_cast<size_t>(xrow[r]) * xstride +
                                                      static_cast<size_t>(sb * 8 + s) * kQ8Bytes);
#pragma unroll
    for (int k = 0; k < 5; ++k) F.xu[r][k] = src[k];
  }
  if constexpr (FMT == QMM_Q4_K) {
    const uint8_t* blk = wr + static_cast<size_t>(sb) * kQ4Bytes;
    F.hdr = ld16_a16(blk);
#pragma unroll
    for (int p = 0; p < 4; ++p) F.q[p] = ld16_a16(blk + 16 + 32 * p + 16 * g);
  } else {
    const uint8_t* blk = wr + static_cast<size_t>(sb) * kQ6Bytes;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        raw8_load(blk + 128 + 32 * h + 16 * hf + 8 * g, F.qh_raw[h][hf], F.sh);
#pragma unroll
        for (int par = 0; par < 2; ++par)
          raw8_load(blk + 64 * h + 32 * par + 16 * hf + 8 * g, F.ql_raw[h][par][hf], F.sh);
      }
    raw8_load(blk + 192 + 8 * g, F.sc_raw, F.sh);
    F.d_raw = ld_u16(blk + 208);
  }
}

// Write super-block sb's prefetched data to LDS stage `st`: activation
// payload, (beta, -beta*C), beta*S, and this wave's decoded weight scales.
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void mmq_commit(const MmqParams& P, uint8_t* st, const MmqPrefetch<FMT, NT>& F,
                                           const int* orow, const bool* cvalid, int sb, int wave, int col,
                                           int g, bool write_dbg_s) {
  using L = MmqSmem<FMT, NT>;
  constexpr int BN = L::BN;
#pragma unroll
  for (int r = 0; r < MmqPrefetch<FMT, NT>::RX; ++r) {
    const int bi = threadIdx.x + kMmqThreads * r;
    const int j = bi >> 3, s = bi & 7;
    const uint2* u = F.xu[r];  // u[0].x = d and pad, u[0].y .. u[4].x = q[0..31], u[4].y = S
    uint8_t* dq = st + L::kXq + s * L::kXqRow;
    if constexpr (FMT == QMM_Q4_K) {
      reinterpret_cast<uint4*>(dq)[j] = make_uint4(u[0].y, u[1].x, u[1].y, u[2].x);
      reinterpret_cast<uint4*>(dq + 16 * BN)[j] = make_uint4(u[2].y, u[3].x, u[3].y, u[4].x);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        reinterpret_cast<uint2*>(dq + 8 * BN * k)[j] = make_uint2(u[k].y, u[k + 1].x);  // q[8k .. 8k+7]
    }
    const float beta = h2f(u[0].x & 0xffffu);
    reinterpret_cast<float2*>(st + L::kXb)[s * L::kXbRow + j] = make_float2(beta, -beta * kMagic);
    if constexpr (FMT == QMM_Q4_K) {
      const int S = static_cast<int>(u[4].y);
      reinterpret_cast<float*>(st + L::kXs)[s * L::kXsRow + j] = beta * static_cast<float>(S);
      if (MODE == kDebug && write_dbg_s && cvalid[r])
        P.dbgS[static_cast<size_t>(orow[r]) * P.nb * 8 + sb * 8 + s] = S;
    }
  }
  float* wa_w = reinterpret_cast<float*>(st + L::kWa) + wave * L::NS16 * 32;
  if constexpr (FMT == QMM_Q4_K) {
    // lane (row col, half g) decodes sub-blocks 4g .. 4g+3 of its row
    const float d = h2f(F.hdr.x & 0xffffu), dmin = h2f(F.hdr.x >> 16);
    float* wm_w = reinterpret_cast<float*>(st + L::kWm) + wave * 8 * 32;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      int sc, m;
      q4k_scale_min(4 * g + jj, F.hdr.y, F.hdr.z, F.hdr.w, sc, m);
      wa_w[(4 * g + jj) * 32 + col] = d * static_cast<float>(sc);
      wm_w[(4 * g + jj) * 32 + col] = -(dmin * static_cast<float>(m));
    }
  } else {
    // lane (row col, half g) holds scales 8g .. 8g+7 of its row
    const float d = h2f(F.d_raw);
    const uint2 sc8 = raw8_join(F.sc_raw, F.sh);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t word = q < 4 ? sc8.x : sc8.y;
      wa_w[(8 * g + q) * 32 + col] = d * static_cast<float>(static_cast<int8_t>((word >> (8 * (q & 3))) & 0xffu));
    }
  }
}

// Store a wave's 32 x (32*NT) fp32 tile.  acc[ct][v] holds row
// 8*(v/4) + 4*(lane/32) + v%4 of the wave's rows and column ct*32 + lane%32.
template <int NT, int MODE>
__device__ __forceinline__ void store_tile(const MmqParams& P, const TileCols& tc, int r0,
                                           const v16f (&acc)[NT], float* out) {
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    int xrow, orow;
    bool valid;
    col_rows<MODE>(P, tc, ct * 32 + col, xrow, orow, valid);
    if (!valid) continue;
    float* yr = out + static_cast<size_t>(orow) * P.M;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = r0 + 8 * k + 4 * g;
      if ((P.M & 3) == 0 && row + 3 < P.M) {
        *reinterpret_cast<float4*>(yr + row) =
            make_float4(acc[ct][4 * k], acc[ct][4 * k + 1], acc[ct][4 * k + 2], acc[ct][4 * k + 3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (row + r < P.M) yr[row + r] = acc[ct][4 * k + r];
      }
    }
  }
}

// A operand bytes of one super-block for this lane (row col of the wave's
// 32 rows, k-group g), taken out of the prefetch registers before the loads
// of the next super-block reuse them.
template <int FMT>
struct MmqOperand;
template <>
struct MmqOperand<QMM_Q4_K> {
  uint4 q[4];  // bytes 16 + 32p + 16g .. +15 of the block: nibbles of sub-blocks 2p, 2p+1
};
template <>
struct MmqOperand<QMM_Q6_K> {
  uint2 ql[2][2][2], qh[2][2];  // [h][parity][16-half] low-nibble bytes, [h][16-half] high-bit bytes
};

template <int FMT, int NT>
__device__ __forceinline__ void take_operand(const MmqPrefetch<FMT, NT>& F, MmqOperand<FMT>& A) {
  if constexpr (FMT == QMM_Q4_K) {
#pragma unroll
    for (int p = 0; p < 4; ++p) A.q[p] = F.q[p];
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        A.qh[h][hf] = raw8_join(F.qh_raw[h][hf], F.sh);
#pragma unroll
        for (int par = 0; par < 2; ++par) A.ql[h][par][hf] = raw8_join(F.ql_raw[h][par][hf], F.sh);
      }
  }
}

// LDS operands of one MFMA sub-block u for this lane: the 16 row scales
// alpha of its rows, (beta, -beta*C) and the B operand of each column tile,
// and for Q4_K at odd u the min-term operands of sub-blocks u-1, u.
template <int FMT, int NT>
struct SubOps {
  using BQ = std::conditional_t<FMT == QMM_Q4_K, v4i, long>;
  float al[16];
  float2 bp[NT];
  BQ bq[NT];
  float am, bm[NT];
};

// u indexes MFMA sub-blocks: Q4_K u = the 32-weight sub-block (= Q8_1 block);
// Q6_K u = 2*s + hf, 16-weight group hf of Q8_1 block s.
template <int FMT, int NT>
__device__ __forceinline__ void load_sub(const uint8_t* st, int u, SubOps<FMT, NT>& O) {
  using L = MmqSmem<FMT, NT>;
  constexpr int BN = L::BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  const int s = FMT == QMM_Q4_K ? u : u >> 1;
  // B operand: piece g (Q4_K: k-group g of the 32 values) or quarter 2*hf+g (Q6_K)
  const uint8_t* xq = st + L::kXq + s * L::kXqRow + L::kPiece * col;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    if constexpr (FMT == QMM_Q4_K)
      O.bq[ct] = *reinterpret_cast<const v4i*>(xq + 16 * BN * g + 16 * 32 * ct);
    else
      O.bq[ct] = *reinterpret_cast<const long*>(xq + 8 * BN * (2 * (u & 1) + g) + 8 * 32 * ct);
  }
  const float* wa = reinterpret_cast<const float*>(st + L::kWa) + wave * L::NS16 * 32 + u * 32 + 4 * g;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 t4 = *reinterpret_cast<const float4*>(wa + 8 * k);
    O.al[4 * k] = t4.x; O.al[4 * k + 1] = t4.y; O.al[4 * k + 2] = t4.z; O.al[4 * k + 3] = t4.w;
  }
  const float2* xb = reinterpret_cast<const float2*>(st + L::kXb) + s * L::kXbRow + col;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) O.bp[ct] = xb[32 * ct];
  if constexpr (FMT == QMM_Q4_K) {
    if (u & 1) {
      O.am = reinterpret_cast<const float*>(st + L::kWm)[wave * 8 * 32 + (u - 1 + g) * 32 + col];
      const float* xs = reinterpret_cast<const float*>(st + L::kXs) + (u - 1 + g) * L::kXsRow + col;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) O.bm[ct] = xs[32 * ct];
    }
  }
}

// A operand of MFMA sub-block u from this lane's weight bytes.
//   Q4_K: the 4-bit values (0..15) of sub-block u, 16 per lane.
//   Q6_K: the signed values q - 32, 8 per lane: the low nibble from ql and
//   the two high bits from qh; a byte-table lookup (v_perm) maps the high
//   bits hi to the int8 16*(hi-2), which has a zero low nibble.
__device__ __forceinline__ v4i build_a(const MmqOperand<QMM_Q4_K>& A, int u) {
  const uint4 qv = A.q[u >> 1];
  const int sh = (u & 1) * 4;
  return v4i{static_cast<int>((qv.x >> sh) & 0x0f0f0f0fu), static_cast<int>((qv.y >> sh) & 0x0f0f0f0fu),
             static_cast<int>((qv.z >> sh) & 0x0f0f0f0fu), static_cast<int>((qv.w >> sh) & 0x0f0f0f0fu)};
}
constexpr uint32_t kQ6HiTable = 0x1000F0E0u;  // bytes -32, -16, 0, 16 as int8
__device__ __forceinline__ long build_a(const MmqOperand<QMM_Q6_K>& A, int u) {
  const int s = u >> 1, hf = u & 1;
  const int h = s >> 2, gg = s & 3, par = gg & 1, shl = 4 * (gg >> 1), shh = 2 * gg;
  const uint2 lq = A.ql[h][par][hf];
  const uint2 hq = A.qh[h][hf];
  const uint32_t q0 = ((lq.x >> shl) & 0x0f0f0f0fu) |
                      __builtin_amdgcn_perm(kQ6HiTable, kQ6HiTable, (hq.x >> shh) & 0x03030303u);
  const uint32_t q1 = ((lq.y >> shl) & 0x0f0f0f0fu) |
                      __builtin_amdgcn_perm(kQ6HiTable, kQ6HiTable, (hq.y >> shh) & 0x03030303u);
  return static_cast<long>((static_cast<unsigned long>(q1) << 32) | q0);
}

__device__ __forceinline__ v16i mfma_sub(const v4i& a, const v4i& b, const v16i& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16i mfma_sub(long a, long b, const v16i& c) {
  return __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, c, 0, 0, 0);
}

// Multiply-accumulate super-block sb from LDS stage st.  Software pipeline
// over sub-blocks: the LDS operands of sub-block u+1 are read while u is
// rescaled, and the MFMA of (u+1, column tile ct) is issued right after the
// epilogue of (u, ct) has consumed its registers, so the matrix core runs
// under the epilogue of the next column tile.  The epilogue adds
// alpha * beta * D into acc (2 VALU ops per element); the Q4_K min term
// goes through fp32 MFMAs into the same accumulator.  Q6_K has no separate
// term: its A operand is already signed.
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void mmq_compute(const MmqParams& P, const uint8_t* st, const MmqOperand<FMT>& A,
                                            v16f (&acc)[NT], const v16i& magic,
                                            const TileCols& tc, int r0, int sb) {
  constexpr int NU = FMT == QMM_Q4_K ? 8 : 16;  // MFMA sub-blocks per super-block
  const int g = (threadIdx.x & 63) >> 5, col = threadIdx.x & 31;
  SubOps<FMT, NT> O[2];
  v16i X[NT];
  load_sub<FMT, NT>(st, 0, O[0]);
  {
    const auto a0 = build_a(A, 0);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) X[ct] = mfma_sub(a0, O[0].bq[ct], magic);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int b = u & 1;
    const bool more = u + 1 < NU;
    if (more) load_sub<FMT, NT>(st, u + 1, O[b ^ 1]);
    const auto an = build_a(A, more ? u + 1 : u);
    // scheduling barriers pin the order: operand reads of u+1 first, then
    // per column tile its epilogue followed by its next MFMA (left to
    // itself the compiler sinks the reads behind the epilogue and exposes
    // the LDS latency)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      if constexpr (MODE == kDebug) {
        int xr, orr; bool ok;
        col_rows<MODE>(P, tc, ct * 32 + col, xr, orr, ok);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = r0 + 8 * (v >> 2) + 4 * g + (v & 3);
          if (ok && row < P.M)
            P.dbgD[(static_cast<size_t>(orr) * P.M + row) * (P.nb * NU) + sb * NU + u] =
                X[ct][v] - static_cast<int>(kMagicBits);
        }
      } else {
        // the whole vector is reinterpreted: X holds 1.5*2^23 + D as fp32 bits
        const v16f Xf = __builtin_bit_cast(v16f, X[ct]);
        const float2 bp = O[b].bp[ct];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float t = __builtin_fmaf(bp.x, Xf[v], bp.y);
          acc[ct][v] = __builtin_fmaf(O[b].al[v], t, acc[ct][v]);
        }
      }
      if constexpr (FMT == QMM_Q4_K && MODE != kDebug) {
        // min term, K = 2 fp32 MFMA over sub-blocks u-1, u (lane half g
        // takes u-1+g): A[i][k] = -dmin*m, B[k][j] = beta*S.  The next VALU
        // write of acc[ct] comes one column tile later, under which it runs.
        if (u & 1) acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(O[b].am, O[b].bm[ct], acc[ct], 0, 0, 0);
      }
      if (more) X[ct] = mfma_sub(an, O[b ^ 1].bq[ct], magic);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Per-thread addressing of one tile: the activation rows this thread stages
// (columns (threadIdx.x + 256 r) / 8) and the weight row of its A operand.
template <int FMT, int NT, int MODE>
struct TileRef {
  static constexpr int RX = MmqPrefetch<FMT, NT>::RX;
  TileCols tc;
  int r0;                 // first row of this wave
  const uint8_t* wr;      // weight row of this lane
  int xrow[RX], orow[RX];
  bool cvalid[RX];
  bool dbg_s;             // debug: this tile writes the activation sums
};

// MoE tables copied to LDS at kernel start: the tile search runs in LDS
// instead of as a chain of dependent global loads.
struct MoeTables {
  const int* work_off;  // [E+1]
  const int* counts;    // [E]
  const int* offsets;   // [E]
};

// Tile idx of the call: rows, routed columns and weight matrix.
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void tile_ref(const MmqParams& P, const MoeTables& Tb, int idx,
                                         TileRef<FMT, NT, MODE>& R) {
  constexpr int BN = 32 * NT;
  int m_tile;
  const uint8_t* wbase = P.w;
  if constexpr (MODE == kMoe) {
    int lo = 0, hi = P.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (Tb.work_off[mid] <= idx) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int cnt = Tb.counts[e];
    const int ntile = (cnt + BN - 1) / BN;
    const int local = idx - Tb.work_off[e];
    m_tile = local / ntile;
    const int n_tile = local % ntile;
    R.tc.n0 = n_tile * BN;
    R.tc.ncols = min(BN, cnt - R.tc.n0);
    R.tc.slot_base = Tb.offsets[e];
    wbase = P.w + static_cast<size_t>(e) * static_cast<size_t>(P.expert_stride);
  } else {
    const int ntile = (P.T + BN - 1) / BN;
    m_tile = idx / ntile;
    const int n_tile = idx % ntile;
    R.tc.n0 = n_tile * BN;
    R.tc.ncols = min(BN, P.T - R.tc.n0);
    R.tc.slot_base = 0;
  }
  R.dbg_s = MODE == kDebug && m_tile == 0;
  R.r0 = m_tile * kMmqBM + (threadIdx.x >> 6) * 32;
  const int wrow = min(R.r0 + (threadIdx.x & 31), P.M - 1);
  constexpr int kRowBytes = FMT == QMM_Q4_K ? kQ4Bytes : kQ6Bytes;
  R.wr = wbase + static_cast<size_t>(wrow) * P.nb * kRowBytes;
#pragma unroll
  for (int r = 0; r < R.RX; ++r)
    col_rows<MODE>(P, R.tc, (threadIdx.x + kMmqThreads * r) >> 3, R.xrow[r], R.orow[r], R.cvalid[r]);
}

// Next tile for this workgroup, or -1 (thread 0 only).  The tiles are split
// into kXcds contiguous ranges with one counter each; a workgroup starts on
// the range of its XCD (blockIdx % kXcds) and moves on when it is drained.
__device__ __forceinline__ int claim_tile(const MmqParams& P, int total, int home, int& qi) {
  for (; qi < kXcds; ++qi) {
    const int q = (home + qi) % kXcds;
    const int start = static_cast<int>((static_cast<int64_t>(total) * q) / kXcds);
    const int size = static_cast<int>((static_cast<int64_t>(total) * (q + 1)) / kXcds) - start;
    const unsigned c = atomicAdd(&P.counters[q], 1u);
    if (c < static_cast<unsigned>(size)) return start + static_cast<int>(c);
  }
  return -1;
}

// Persistent loop over the tiles of the call, software-pipelined over
// super-blocks: while super-block k is multiplied from LDS stage k&1, the
// loads of super-block k+1 are in flight, across tile boundaries too.  One
// barrier per super-block: the write of stage (k+1)&1 comes after the
// barrier of k, which every wave passes only after finishing super-block
// k-1 from that stage.  Tiles are claimed two ahead: thread 0 issues the
// claim of tile i+2 at the first super-block of tile i and publishes it in
// a 3-slot ring at the end of tile i, so neither the atomic's latency nor
// the next tile's set-up waits in front of a barrier.  Two waves per SIMD
// are required: with one, nothing hides the MFMA and LDS latencies of the
// epilogue.
template <int FMT, int NT, int MODE>
__global__ __launch_bounds__(kMmqThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mmq_kernel(MmqParams P) {
  using L = MmqSmem<FMT, NT>;
  constexpr int BN = L::BN;
  constexpr int kTab = MODE == kMoe ? kMoeMaxE + 1 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];
  __shared__ int s_tile[3];
  __shared__ int s_work_off[kTab], s_counts[kTab], s_offsets[kTab];

  MoeTables Tb{s_work_off, s_counts, s_offsets};
  int total;
  if constexpr (MODE == kMoe) {
    for (int i = threadIdx.x; i <= P.E; i += kMmqThreads) {
      s_work_off[i] = P.work_off[i];
      if (i < P.E) {
        s_counts[i] = P.counts[i];
        s_offsets[i] = P.offsets[i];
      }
    }
    total = P.work_off[P.E];
  } else {
    total = ((P.M + kMmqBM - 1) / kMmqBM) * ((P.T + BN - 1) / BN);
  }
  const int home = static_cast<int>(blockIdx.x % kXcds);
  int qi = 0;  // queue cursor, used by thread 0 only
  if (threadIdx.x == 0) {
    s_tile[0] = claim_tile(P, total, home, qi);
    s_tile[1] = s_tile[0] >= 0 ? claim_tile(P, total, home, qi) : -1;
  }
  __syncthreads();
  int cur = s_tile[0];
  if (cur >= 0) {
    const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31, wave = threadIdx.x >> 6;
    const size_t xstride = static_cast<size_t>(P.nb) * 8 * kQ8Bytes;
    v16i magic;
#pragma unroll
    for (int v = 0; v < 16; ++v) magic[v] = static_cast<int>(kMagicBits);
    TileRef<FMT, NT, MODE> R, Rn;
    tile_ref<FMT, NT, MODE>(P, Tb, cur, R);
    MmqPrefetch<FMT, NT> F;
    mmq_load<FMT, NT>(P, F, R.xrow, xstride, R.wr, 0, g);
    int k = 0;        // super-blocks done by this workgroup (selects the LDS stage)
    int pending = -1;  // thread 0: claim in flight for tile it+2
    for (int it = 0;; ++it) {
      v16f acc[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ct][v] = 0.0f;
      int next = -1;
      for (int sb = 0; sb < P.nb; ++sb, ++k) {
        uint8_t* st = smem + (k & 1) * L::kStage;
        mmq_commit<FMT, NT, MODE>(P, st, F, R.orow, R.cvalid, sb, wave, col, g, R.dbg_s);
        MmqOperand<FMT> A;
        take_operand<FMT, NT>(F, A);
        __syncthreads();
        if (sb == 0) {
          // tile it+1 was published before this barrier; its rows resolve
          // under this tile's super-blocks
          next = s_tile[(it + 1) % 3];
          if (next >= 0) tile_ref<FMT, NT, MODE>(P, Tb, next, Rn);
          if (threadIdx.x == 0) pending = next >= 0 ? claim_tile(P, total, home, qi) : -1;
        }
        if (sb + 1 < P.nb) {
          mmq_load<FMT, NT>(P, F, R.xrow, xstride, R.wr, sb + 1, g);
        } else if (next >= 0) {
          mmq_load<FMT, NT>(P, F, Rn.xrow, xstride, Rn.wr, 0, g);
        }
        mmq_compute<FMT, NT, MODE>(P, st, A, acc, magic, R.tc, R.r0, sb);
      }
      if constexpr (MODE != kDebug) store_tile<NT, MODE>(P, R.tc, R.r0, acc, P.y);
      if (next < 0) break;
      R = Rn;
      // slot (it+2)%3 was last read at the first barrier of tile it-1
      if (threadIdx.x == 0) s_tile[(it + 2) % 3] = pending;
    }
  }
  // exit: the last workgroup out resets the queue counters for the next call
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned done = atomicAdd(&P.counters[kXcds], 1u);
    if (done == gridDim.x - 1) {
      for (int q = 0; q < kXcds; ++q) atomicExch(&P.counters[q], 0u);
      atomicExch(&P.counters[kXcds], 0u);
    }
  }
}

// Grid size: enough resident workgroups to fill the device, a multiple of
// the XCD count so every XCD range has workers.
template <int FMT, int NT, int MODE>
static int mmq_grid(int total_tiles_hint) {
  static int per_cu = -1;
  if (per_cu < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mmq_kernel<FMT, NT, MODE>, kMmqThreads, 0) !=
            hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  int g = device_cu_count() * per_cu;
  if (total_tiles_hint > 0 && total_tiles_hint < g) g = total_tiles_hint;
  g = ((g + kXcds - 1) / kXcds) * kXcds;
  return g < kXcds ? kXcds : g;
}

template <int FMT, int NT, int MODE>
static int launch_mmq(const MmqParams& P, int total_tiles_hint, hipStream_t st) {
  const int grid = mmq_grid<FMT, NT, MODE>(total_tiles_hint);
  hipLaunchKernelGGL((mmq_kernel<FMT, NT, MODE>), dim3(grid), dim3(kMmqThreads), 0, st, P);
  return launch_status();
}

constexpr int kMoeNT = 1;    // MoE tiles: 128 rows x 32 routed tokens
constexpr size_t kCounterBytes = 256;

// Dense tiles are 128 rows x 64 tokens, or 128 x 32 when there are very few
// 64-token tiles.  (A 64-token tile per CU outruns two 32-token tiles per
// CU: the A operand, row scales and epilogue set-up are shared by twice the
// MFMAs.)
constexpr int64_t kDenseMinTiles2 = 64;
template <int FMT>
static int mmq_dense_fmt(const MmqParams& P, bool dbg, hipStream_t st) {
  const int64_t mt = (P.M + kMmqBM - 1) / kMmqBM;
  const int64_t tiles2 = mt * ((P.T + 63) / 64);
  if (tiles2 >= kDenseMinTiles2)
    return dbg ? launch_mmq<FMT, 2, kDebug>(P, static_cast<int>(tiles2), st)
               : launch_mmq<FMT, 2, kDense>(P, static_cast<int>(tiles2), st);
  const int tiles1 = static_cast<int>(mt * ((P.T + 31) / 32));
  return dbg ? launch_mmq<FMT, 1, kDebug>(P, tiles1, st) : launch_mmq<FMT, 1, kDense>(P, tiles1, st);
}

int mmq_dense(int fmt, const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
              void* ws, hipStream_t st, int32_t* dbgD, int32_t* dbgS) {
  MmqParams P{};
  P.w = static_cast<const uint8_t*>(w);
  P.xq = static_cast<const uint8_t*>(xq);
  P.y = y;
  P.M = static_cast<int>(M);
  P.nb = static_cast<int>(K / kQK);
  P.T = static_cast<int>(T);
  P.counters = static_cast<unsigned*>(ws);
  P.dbgD = dbgD;
  P.dbgS = dbgS;
  const bool dbg = dbgD != nullptr;
  return fmt == QMM_Q4_K ? mmq_dense_fmt<QMM_Q4_K>(P, dbg, st) : mmq_dense_fmt<QMM_Q6_K>(P, dbg, st);
}

// Grouped launch used by moe_grouped_mmq (after route preparation on the
// same stream): tiles of 128 rows x 32 routed slots.
int mmq_moe_launch(int fmt, const uint8_t* w, int64_t stride, int M, int nb, const uint8_t* xq,
                   float* out, unsigned* counters, const int32_t* counts, const int32_t* offsets,
                   const int32_t* bucket, const int32_t* work_off, int E, int top_k,
                   int rows_per_token, hipStream_t st) {
  static_assert(32 * kMoeNT == 32 && kMmqBM == 128, "route preparation assumes 128 x 32 tiles");
  MmqParams P{};
  P.w = w;
  P.xq = xq;
  P.y = out;
  P.M = M;
  P.nb = nb;
  P.T = 0;
  P.counters = counters;
  P.counts = counts;
  P.offsets = offsets;
  P.bucket = bucket;
  P.work_off = work_off;
  P.E = E;
  P.top_k = top_k;
  P.rows_per_token = rows_per_token;
  P.expert_stride = stride;
  if (fmt == QMM_Q4_K) return launch_mmq<QMM_Q4_K, kMoeNT, kMoe>(P, 0, st);
  return launch_mmq<QMM_Q6_K, kMoeNT, kMoe>(P, 0, st);
}

static int check_mmq(const void* w, const void* xq, const float* y, int64_t M, int64_t K, int64_t T,
                     const void* ws, size_t ws_bytes) {
  if (M < 1 || T < 1 || K < kQK || (K % kQK) != 0) return QMM_ERR_SHAPE;
  if (M > (1 << 30) || T > (1 << 30) || K / kQK > (1 << 20)) return QMM_ERR_SHAPE;
  if (!w || !xq || !y || !ws) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(y) || !aligned16(ws)) return QMM_ERR_ALIGN;
  if (ws_bytes < kCounterBytes) return QMM_ERR_WORKSPACE;
  return QMM_OK;
}

}  // namespace qmm

using namespace qmm;

extern "C" int mmq_q4k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                       void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, xq, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q4_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr);
}

extern "C" int mmq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                       void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, xq, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q6_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr);
}
