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
// consecutive.  Rows of s are padded so that the commit stores (8 lanes =
// the 8 blocks of one token) fall on different banks; reads stay a per-lane
// base plus immediate offsets.
template <int FMT, int NT>
struct MmqSmem {
  static constexpr int BN = 32 * NT;
  static constexpr int NS16 = FMT == QMM_Q4_K ? 8 : 16;     // scale groups per super-block
  static constexpr int kPiece = FMT == QMM_Q4_K ? 16 : 8;    // payload bytes per piece
  static constexpr int kXqRow = 32 * BN + 8 * kPiece;       // bytes per block row s
  static constexpr int kXbRow = BN + 8;                      // float2 per block row
  static constexpr int kXsRow = FMT == QMM_Q4_K ? BN + 8 : BN + 4;  // floats per scale row
  static constexpr int kXq = 0;                              // [8][32/kPiece][BN][kPiece] int8 payload
  static constexpr int kXb = kXq + 8 * kXqRow;               // [8][kXbRow] (beta, -beta*C)
  static constexpr int kXs = kXb + 8 * kXbRow * 8;           // [NS16][kXsRow] beta*S (Q4_K: per 32, Q6_K: per 16)
  static constexpr int kWa = kXs + NS16 * kXsRow * 4;        // [4 waves][NS16][32] alpha = d*sc
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
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(a & ~static_cast<uintptr_t>(3));
  sh = static_cast<uint32_t>(a & 3u);
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
    } else {
      int S0 = dot4(0x01010101u, u[0].y, 0);
      S0 = dot4(0x01010101u, u[1].x, S0);
      S0 = dot4(0x01010101u, u[1].y, S0);
      S0 = dot4(0x01010101u, u[2].x, S0);
      int S1 = dot4(0x01010101u, u[2].y, 0);
      S1 = dot4(0x01010101u, u[3].x, S1);
      S1 = dot4(0x01010101u, u[3].y, S1);
      S1 = dot4(0x01010101u, u[4].x, S1);
      float* xs = reinterpret_cast<float*>(st + L::kXs);
      xs[(2 * s) * L::kXsRow + j] = beta * static_cast<float>(S0);
      xs[(2 * s + 1) * L::kXsRow + j] = beta * static_cast<float>(S1);
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

// One output tile: rows [m0, m0+128) of weight matrix wbase, columns tc.
// Software pipeline over super-blocks: while super-block sb is multiplied
// from LDS stage sb&1, the loads of sb+1 are in flight; one barrier per
// super-block (the double buffer makes the write of stage (sb+1)&1 safe:
// every wave has passed the barrier of sb, hence finished reading sb-1).
// Within a super-block the MFMAs of one sub-block are issued together, then
// their epilogues; scheduling barriers between sub-blocks keep later MFMAs
// from being hoisted (their results would not fit in registers).
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void mmq_tile(const MmqParams& P, uint8_t* smem, const uint8_t* wbase,
                                         int m0, const TileCols& tc, bool write_dbg_s) {
  using L = MmqSmem<FMT, NT>;
  constexpr int BN = L::BN;
  constexpr int RX = MmqPrefetch<FMT, NT>::RX;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  const int r0 = m0 + wave * 32;
  const int wrow = min(r0 + col, P.M - 1);  // A-operand row of this lane
  const size_t xstride = static_cast<size_t>(P.nb) * 8 * kQ8Bytes;
  constexpr int kRowBytes = FMT == QMM_Q4_K ? kQ4Bytes : kQ6Bytes;
  const uint8_t* wr = wbase + static_cast<size_t>(wrow) * P.nb * kRowBytes;

  int xrow[RX], orow[RX];
  bool cvalid[RX];
#pragma unroll
  for (int r = 0; r < RX; ++r)
    col_rows<MODE>(P, tc, (threadIdx.x + kMmqThreads * r) >> 3, xrow[r], orow[r], cvalid[r]);

  v16f acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ct][v] = 0.0f;
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = static_cast<int>(kMagicBits);

  MmqPrefetch<FMT, NT> F;
  mmq_load<FMT, NT>(P, F, xrow, xstride, wr, 0, g);
  for (int sb = 0; sb < P.nb; ++sb) {
    uint8_t* st = smem + (sb & 1) * L::kStage;
    mmq_commit<FMT, NT, MODE>(P, st, F, orow, cvalid, sb, wave, col, g, write_dbg_s);
    // this super-block's A operand bytes leave the prefetch registers
    uint4 qcur[4];
    uint2 qlc[2][2][2], qhc[2][2];
    if constexpr (FMT == QMM_Q4_K) {
#pragma unroll
      for (int p = 0; p < 4; ++p) qcur[p] = F.q[p];
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          qhc[h][hf] = raw8_join(F.qh_raw[h][hf], F.sh);
#pragma unroll
          for (int par = 0; par < 2; ++par) qlc[h][par][hf] = raw8_join(F.ql_raw[h][par][hf], F.sh);
        }
    }
    __syncthreads();
    if (sb + 1 < P.nb) mmq_load<FMT, NT>(P, F, xrow, xstride, wr, sb + 1, g);

    const float* wa = reinterpret_cast<const float*>(st + L::kWa) + wave * L::NS16 * 32;
    const uint8_t* xqs = st + L::kXq;
    const float2* xb = reinterpret_cast<const float2*>(st + L::kXb);
    const float* xs = reinterpret_cast<const float*>(st + L::kXs);

    if constexpr (FMT == QMM_Q4_K) {
      const float* wm = reinterpret_cast<const float*>(st + L::kWm) + wave * 8 * 32;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int p = s >> 1;
        const uint4 qv = qcur[p];
        const int sh = (s & 1) * 4;
        const v4i a = {static_cast<int>((qv.x >> sh) & 0x0f0f0f0fu), static_cast<int>((qv.y >> sh) & 0x0f0f0f0fu),
                       static_cast<int>((qv.z >> sh) & 0x0f0f0f0fu), static_cast<int>((qv.w >> sh) & 0x0f0f0f0fu)};
        v16i X[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const v4i bq = *reinterpret_cast<const v4i*>(xqs + s * L::kXqRow + 16 * BN * g + 16 * (ct * 32 + col));
          X[ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, magic, 0, 0, 0);
        }
        float al[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 t4 = *reinterpret_cast<const float4*>(wa + s * 32 + 8 * k + 4 * g);
          al[4 * k] = t4.x; al[4 * k + 1] = t4.y; al[4 * k + 2] = t4.z; al[4 * k + 3] = t4.w;
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const int jcol = ct * 32 + col;
          if constexpr (MODE == kDebug) {
            int xr, orr; bool ok;
            col_rows<MODE>(P, tc, jcol, xr, orr, ok);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int row = r0 + 8 * (v >> 2) + 4 * g + (v & 3);
              if (ok && row < P.M)
                P.dbgD[(static_cast<size_t>(orr) * P.M + row) * (P.nb * 8) + sb * 8 + s] =
                    X[ct][v] - static_cast<int>(kMagicBits);
            }
          } else {
            const float2 bp = xb[s * L::kXbRow + jcol];
            // the whole vector is reinterpreted: X holds 1.5*2^23 + D as fp32 bits
            const v16f Xf = __builtin_bit_cast(v16f, X[ct]);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float t = __builtin_fmaf(bp.x, Xf[v], bp.y);
              acc[ct][v] = __builtin_fmaf(al[v], t, acc[ct][v]);
            }
          }
        }
        if (s & 1) {
          // min term of sub-blocks s-1, s: A[i][k] = -dmin*m, B[k][j] = beta*S
          const float am = wm[(s - 1 + g) * 32 + col];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const float bm = xs[(s - 1 + g) * L::kXsRow + ct * 32 + col];
            acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(am, bm, acc[ct], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {  // Q8_1 block = 32-group (h = s/4, gg = s%4)
        const int h = s >> 2, gg = s & 3, par = gg & 1, shl = 4 * (gg >> 1), shh = 2 * gg;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint2 lq = qlc[h][par][hf];
          const uint2 hq = qhc[h][hf];
          const uint32_t q0 = ((lq.x >> shl) & 0x0f0f0f0fu) | (((hq.x >> shh) & 0x03030303u) << 4);
          const uint32_t q1 = ((lq.y >> shl) & 0x0f0f0f0fu) | (((hq.y >> shh) & 0x03030303u) << 4);
          const long a = static_cast<long>((static_cast<unsigned long>(q1) << 32) | q0);
          const int s16 = 2 * s + hf;
          v16i X[NT];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const long bq = *reinterpret_cast<const long*>(xqs + s * L::kXqRow + 8 * BN * (2 * hf + g) + 8 * (ct * 32 + col));
            X[ct] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, bq, magic, 0, 0, 0);
          }
          float al[16];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float4 t4 = *reinterpret_cast<const float4*>(wa + s16 * 32 + 8 * k + 4 * g);
            al[4 * k] = t4.x; al[4 * k + 1] = t4.y; al[4 * k + 2] = t4.z; al[4 * k + 3] = t4.w;
          }
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) {
            const int jcol = ct * 32 + col;
            if constexpr (MODE == kDebug) {
              int xr, orr; bool ok;
              col_rows<MODE>(P, tc, jcol, xr, orr, ok);
              // D6 = sum (q6 - 32) q = D - 32 * S16, S16 = sum of the 16 int8 activations
              const uint2 p0 = *reinterpret_cast<const uint2*>(xqs + s * L::kXqRow + 8 * BN * (2 * hf) + 8 * jcol);
              const uint2 p1 = *reinterpret_cast<const uint2*>(xqs + s * L::kXqRow + 8 * BN * (2 * hf + 1) + 8 * jcol);
              int S16 = dot4(0x01010101u, p0.x, 0);
              S16 = dot4(0x01010101u, p0.y, S16);
              S16 = dot4(0x01010101u, p1.x, S16);
              S16 = dot4(0x01010101u, p1.y, S16);
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int row = r0 + 8 * (v >> 2) + 4 * g + (v & 3);
                if (ok && row < P.M)
                  P.dbgD[(static_cast<size_t>(orr) * P.M + row) * (P.nb * 16) + sb * 16 + s16] =
                      X[ct][v] - static_cast<int>(kMagicBits) - 32 * S16;
              }
            } else {
              const float2 bp = xb[s * L::kXbRow + jcol];
              const v16f Xf = __builtin_bit_cast(v16f, X[ct]);
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const float t = __builtin_fmaf(bp.x, Xf[v], bp.y);
                acc[ct][v] = __builtin_fmaf(al[v], t, acc[ct][v]);
              }
            }
          }
          if constexpr (MODE != kDebug) {
            if (hf) {
              // offset term of the two 16-halves of block s: A = -32 * d * sc, B = beta * S16
              const float am = -32.0f * wa[(2 * s + g) * 32 + col];
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) {
                const float bm = xs[(2 * s + g) * L::kXsRow + ct * 32 + col];
                acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(am, bm, acc[ct], 0, 0, 0);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  if constexpr (MODE != kDebug) store_tile<NT, MODE>(P, tc, r0, acc, P.y);
}

// Persistent loop over the tiles of the call.  Two waves per SIMD are
// required: with one, nothing hides the MFMA and LDS latencies of the
// epilogue.  (Q6_K with 64-column tiles then spills a few registers to
// scratch, which costs less than one resident wave or 32-column tiles.)
template <int FMT, int NT, int MODE>
__global__ __launch_bounds__(kMmqThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mmq_kernel(MmqParams P) {
  using L = MmqSmem<FMT, NT>;
  constexpr int BN = L::BN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];
  __shared__ unsigned s_claim;

  const int mt = (P.M + kMmqBM - 1) / kMmqBM;
  int total;
  if constexpr (MODE == kMoe) {
    total = P.work_off[P.E];
  } else {
    total = mt * ((P.T + BN - 1) / BN);
  }
  const int home = static_cast<int>(blockIdx.x % kXcds);
  for (int qi = 0; qi < kXcds; ++qi) {
    const int q = (home + qi) % kXcds;
    const int start = static_cast<int>((static_cast<int64_t>(total) * q) / kXcds);
    const int size = static_cast<int>((static_cast<int64_t>(total) * (q + 1)) / kXcds) - start;
    while (true) {
      if (threadIdx.x == 0) s_claim = atomicAdd(&P.counters[q], 1u);
      __syncthreads();
      const unsigned c = s_claim;
      __syncthreads();
      if (c >= static_cast<unsigned>(size)) break;
      const int idx = start + static_cast<int>(c);
      TileCols tc;
      int m_tile;
      const uint8_t* wbase = P.w;
      if constexpr (MODE == kMoe) {
        int lo = 0, hi = P.E;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (P.work_off[mid] <= idx) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int cnt = P.counts[e];
        const int ntile = (cnt + BN - 1) / BN;
        const int local = idx - P.work_off[e];
        m_tile = local / ntile;
        const int n_tile = local % ntile;
        tc.n0 = n_tile * BN;
        tc.ncols = min(BN, cnt - tc.n0);
        tc.slot_base = P.offsets[e];
        wbase = P.w + static_cast<size_t>(e) * static_cast<size_t>(P.expert_stride);
      } else {
        const int ntile = (P.T + BN - 1) / BN;
        m_tile = idx / ntile;
        const int n_tile = idx % ntile;
        tc.n0 = n_tile * BN;
        tc.ncols = min(BN, P.T - tc.n0);
        tc.slot_base = 0;
      }
      mmq_tile<FMT, NT, MODE>(P, smem, wbase, m_tile * kMmqBM, tc, MODE == kDebug && m_tile == 0);
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

// Dense tiles: 128 rows x 64 tokens for both formats.
template <int FMT>
constexpr int kDenseNT = 2;
constexpr int kMoeNT = 1;    // MoE tiles: 128 rows x 32 routed tokens
constexpr size_t kCounterBytes = 256;

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
  const int64_t mt = (M + kMmqBM - 1) / kMmqBM;
  if (fmt == QMM_Q4_K) {
    constexpr int NT = kDenseNT<QMM_Q4_K>;
    const int tiles = static_cast<int>(mt * ((T + 32 * NT - 1) / (32 * NT)));
    return dbg ? launch_mmq<QMM_Q4_K, NT, kDebug>(P, tiles, st) : launch_mmq<QMM_Q4_K, NT, kDense>(P, tiles, st);
  }
  constexpr int NT = kDenseNT<QMM_Q6_K>;
  const int tiles = static_cast<int>(mt * ((T + 32 * NT - 1) / (32 * NT)));
  return dbg ? launch_mmq<QMM_Q6_K, NT, kDebug>(P, tiles, st) : launch_mmq<QMM_Q6_K, NT, kDense>(P, tiles, st);
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
