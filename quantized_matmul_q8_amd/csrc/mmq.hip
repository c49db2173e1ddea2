// Prefill GEMM (MMQ) and its MoE grouped form: y[t][i] = sum_k W[i][k] x_t[k]
// for many tokens, Q4_K, Q5_K or Q6_K weights against Q8_1 activations, on int8
// MFMA with int32 accumulation per sub-block and an fp32 epilogue.
//
// Prior art: [MMQ] "Kernel architecture" (tiles of weights x tokens, dequant
// fused into the matrix inner loop, Q8_1 activations, persistent workgroups
// claiming tiles from an atomic counter instead of Stream-K plus a fixup
// pass, MoE work entries (expert, m_tile, n_tile)); [GAP] root cause 1 and
// lever T1; [8e] §2 for the min-term factorisation.  Re-designed for gfx950:
//
// * Activation repack.  A pre-pass turns the Q8_1 rows of every 32-column
//   tile (tokens; for MoE the routed slots of one expert, gathered through
//   the bucket) into one chunk per super-block: the int8 values in MFMA
//   B-operand order (sub-block s, 16-value half h, column), then per (s,
//   column) the fp32 pair (beta, -beta*C) of the epilogue and beta*S of the
//   min term.  The main kernel then copies whole chunks from global memory
//   straight into LDS (global_load_lds_dwordx4: no registers, no VALU), so
//   staging costs a few instructions per super-block.
// * Matrix core.  One v_mfma_i32_32x32x32_i8 covers one 32-weight Q4_K
//   sub-block of 32 rows x 32 columns: A = unpacked 4-bit values (0..15),
//   B = the Q8_1 int8 values, int32 result D per (row, column, sub-block).
//   Q6_K has 16-weight sub-blocks and uses v_mfma_i32_32x32x16_i8 with the
//   signed values q6 - 32 as A.
// * Epilogue.  Every (row i, column j, sub-block s) has its own factor
//   alpha_is * beta_js, so each MFMA result is rescaled before the next
//   sub-block.  The MFMA accumulator starts at the bits of 1.5*2^23; since
//   |D| < 2^22 the int32 result read as fp32 is exactly 1.5*2^23 + D, and
//     t   = fma(beta, X, -beta*1.5*2^23)   = beta*D, rounded once
//     acc = fma(alpha, t, acc)
//   is two fp32 VALU ops per output element per sub-block.  The Q4_K min
//   term sum_s (-dmin*m_is) * (beta_js*S_js) runs on bf16 MFMA straight into
//   the accumulator: both factors are split exactly into three bf16 parts
//   (-dmin*m has at most 17 significant bits, beta*S at most 23), and six of
//   the nine part products -- all but those below 2^-23 of the whole --
//   make up K = 48 per super-block, three v_mfma_f32_32x32x16_bf16.  The
//   fp32 32x32x2 MFMA it replaces took 64 matrix cycles per two sub-blocks
//   and held the epilogue back by a quarter (ceiling probe: 0.85 against
//   1.0 POP/s).
// * Workgroup.  Eight waves (two per SIMD, which the VALU-bound epilogue
//   needs to reach the issue rate): a tile of 128 rows x 32*NT columns, row
//   group rw = wave % 4 (32 rows), K half kh = wave / 4 taking the
//   super-blocks of parity kh.  The two halves are summed through LDS at the
//   end of the tile, in a fixed order.  One barrier per step of two
//   super-blocks; the next step's chunks and weight bytes are in flight
//   during the current step (double-buffered LDS, register prefetch).
//   With one column tile (MoE tiles, dense calls of up to 32 tokens) the
//   kernel is held to 128 VGPRs instead and runs two workgroups per CU,
//   four waves per SIMD: the other workgroup's work covers a workgroup's
//   barriers and load waits (13-19% faster grouped calls than software
//   pipelining at two waves per SIMD).  Grouped Q4_K / Q5_K calls do not
//   split K: the tile is 256 rows x 32 routed slots, each of the eight waves
//   taking every super-block of its own 32 rows, one super-block per step.
// * Work queue.  Persistent grid, one (one-tile kernel: two) workgroup(s)
//   per CU; tiles are split into
//   8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8), each
//   with its own atomic counter, so a range's weight rows stay in one XCD's
//   L2.  A workgroup's first tile is fixed by its index; later tiles are
//   claimed one ahead, with the atomic's latency hidden under the current
//   tile.  With enough tiles to fill the chip, a tile runs its whole K loop
//   in one workgroup (no fixup).  A dense call with few tiles (few tokens,
//   few rows) splits each tile's K range over up to kMaxSplit workgroups:
//   each writes its fp32 partial tile to the workspace and bumps the tile's
//   arrival counter; the last to arrive adds the partials in split order and
//   stores the tile, so results stay deterministic without float atomics.
//   The kernel that runs just before on the stream (activation repack, route
//   preparation) zeroes the counters, so the workspace needs no
//   initialisation and no memset.
#include "qmm_common.hpp"

#include <mutex>
#include <type_traits>

namespace qmm {

constexpr int kMmqWaves = 8;
constexpr int kMmqThreads = 64 * kMmqWaves;
constexpr int kMmqBM = 128;            // weight rows per tile (32 per row group)
constexpr int kGroupM = 8;             // row tiles per run of the dense tile order

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// x = p0 + p1 + p2 exactly for x with at most 24 significant bits (and no
// bf16 underflow): each part keeps the top 8 bits of what remains.
__device__ __forceinline__ void split3_bf16(float x, __bf16& p0, __bf16& p1, __bf16& p2) {
  p0 = static_cast<__bf16>(x);
  const float r = x - static_cast<float>(p0);
  p1 = static_cast<__bf16>(r);
  p2 = static_cast<__bf16>(r - static_cast<float>(p1));
}

// Min-term MFMA k (0..2), lane half h: partial product j = 2k + h is
// A-part kMinP[j] times B-part kMinQ[j] over the 8 sub-blocks of a
// super-block.  The six pairs are those with p + q <= 2 (the rest are below
// 2^-23 of the product).
__device__ __forceinline__ int min_part_a(int j) { return (0x210100 >> (4 * j)) & 3; }  // 0,0,1,0,1,2
__device__ __forceinline__ int min_part_b(int j) { return (0x012010 >> (4 * j)) & 3; }  // 0,1,0,2,1,0

// Repacked activation chunk: 32 columns x one super-block (8 Q8_1 blocks).
constexpr int kChunkCols = 32;
constexpr int kChunkPay = 0;       // [8 s][2 h][32 col] x 16 bytes: values 16h .. 16h+15 of block s
constexpr int kChunkFac = 8192;    // [8 s][32 col] float2 (beta, -beta*C)
constexpr int kChunkMin = 10240;   // [3 q][32 col][8 s] bf16: part q of beta*S (min-term B operand)
constexpr int kChunkBytes = 12288; // 12 x 1 KB (the last 512 bytes unused)
constexpr int kChunkKB = kChunkBytes / 1024;

enum MmqMode { kDense = 0, kMoe = 1, kDebug = 2, kMoeGlu = 3 };
// kMoeGlu: the grouped gate||up product with SwiGLU -> Q8_1 in the epilogue
template <int MODE>
constexpr bool kIsMoe = MODE == kMoe || MODE == kMoeGlu;

// Q4_K and Q5_K share the kernel's structure (32-weight sub-blocks = Q8_1
// blocks, a 6-bit scale and min per sub-block, the min term); Q5_K adds a
// fifth bit per weight to the A operand.
__host__ __device__ constexpr bool is_q4fam(int fmt) { return fmt == QMM_Q4_K || fmt == QMM_Q5_K; }

// Split-K of dense calls with few tiles: split until about kSplitTiles
// tiles, at most kMaxSplit ways and at least four super-blocks per split.
constexpr int kSplitTiles = 256;
constexpr int kMaxSplit = 16;
// Workspace head: queue counters at word 0, split-K arrival counters (one
// per tile, fewer than kSplitTiles tiles when split) at word 256.
constexpr size_t kCounterBytes = 2048;
constexpr int kTileCntWord = 256;

struct MmqParams {
  const uint8_t* w;
  const uint8_t* xr;            // repacked chunks: (ctile, sb) at (ctile * nb + sb) * kChunkBytes
  float* y;
  int M, nb, T;                 // rows, super-blocks per row, columns (dense)
  unsigned* counters;           // kXcds work-queue counters (zero at kernel start)
  // dense split-K (nsplit == 1: none)
  int nsplit;
  float* part;                  // [tile][split] fp32 partial tiles
  unsigned* tile_cnt;           // [tile] arrival counters (zero at kernel start)
  // MoE (mode kMoe)
  const int32_t* counts;        // [E] routed slots per expert
  const int32_t* offsets;       // [E+1] slot offsets into bucket
  const int32_t* bucket;        // [T*top_k] slots grouped by expert
  const int32_t* ct_off;        // [E+1] prefix of column tiles (chunk rows)
  int mt;                       // row tiles per expert: work entry = mt * ct_off[e] + m_tile * tiles_e + n_tile
  int E;
  int64_t expert_stride;
  // debug (mode kDebug)
  int32_t* dbgD;
  // grouped gate||up with SwiGLU (mode kMoeGlu): gate rows [0, glu_f), up
  // rows [glu_f, 2 glu_f); Q8_1 output rows of glu_f / 32 blocks per slot
  uint8_t* yq;
  int glu_f;
  // fused FFN layer: instead of Q8_1 rows, the down product's activation
  // chunks (its nb_next super-blocks per column tile) go to xr_next
  uint8_t* xr_next;
  int nb_next;
};

// ----------------------------------------------------------------------------
// Activation repack: one workgroup per (super-block sb, column tile); thread
// (s = tid / 32, col = tid % 32) converts block (row of col, 8 sb + s).
// ----------------------------------------------------------------------------
struct RepackParams {
  const uint8_t* xq;
  const float* xf;              // fp32 rows instead of Q8_1 (fused quantizer), or nullptr
  uint8_t* xr;
  int nb;                       // super-blocks per row
  int T;                        // dense: rows
  int ct0;                      // column tile of blockIdx.y == 0 (grid y is launched in chunks)
  // MoE: column tile -> (expert, slots)
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* bucket;
  const int32_t* ct_off;
  int E, top_k, rows_per_token;
  int32_t* dbgS;                // dense debug: S[row][K/32]
  unsigned* counters;           // work-queue counters (and, dense, split-K arrival counters), zeroed here
};

// Activation row of column `col` of chunk row `ctile` (dense: token; MoE:
// the routed slot's row), and the number of valid columns of the chunk row.
// Returns false when the chunk row lies past the routed column tiles.  MoE:
// ct is the column-tile prefix ct_off[0..E] copied to LDS, so the search
// over it is not a chain of dependent global loads.
template <int MODE>
__device__ __forceinline__ bool repack_row(const RepackParams& P, const int* ct, int ctile, int col, int& xrow,
                                           int& ncols) {
  xrow = 0;
  if constexpr (MODE == kMoe) {
    if (ctile >= ct[P.E]) return false;
    int lo = 0, hi = P.E;  // expert e with ct_off[e] <= ctile < ct_off[e+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ct[mid] <= ctile) lo = mid; else hi = mid;
    }
    const int n0 = (ctile - ct[lo]) * kChunkCols;
    ncols = min(kChunkCols, P.counts[lo] - n0);
    if (col < ncols) {
      const int slot = P.bucket[P.offsets[lo] + n0 + col];
      xrow = P.rows_per_token == 1 ? slot / P.top_k : slot;
    }
  } else {
    ncols = min(kChunkCols, P.T - ctile * kChunkCols);
    xrow = ctile * kChunkCols + col;
  }
  return true;
}

// Fused quantizer ([MMQ] "What they do right": activations quantized to
// Q8_1 on the way into the GEMM): the chunk is built from fp32 rows with the
// block quantizer of q8_1_quantize, so its bytes equal those of
// q8_1_quantize followed by the Q8_1 repack.  Eight lanes per block; the 32
// blocks of one pass are 8 consecutive blocks of 4 rows, so a wave reads
// 1 KB of contiguous fp32 per row.
template <int MODE>
__device__ __forceinline__ void repack_f32(const RepackParams& P, const int* ct, int sb, int ctile) {
  __shared__ int s_rows[kChunkCols];
  __shared__ int s_ncols;
  if (threadIdx.x < kChunkCols) {
    int xrow, ncols;
    repack_row<MODE>(P, ct, ctile, threadIdx.x, xrow, ncols);
    s_rows[threadIdx.x] = xrow;
    if (threadIdx.x == 0) s_ncols = ncols;
  }
  __syncthreads();
  const int ncols = s_ncols;
  const int part = threadIdx.x & 7;
  const size_t kf = static_cast<size_t>(P.nb) * kQK;  // floats per row
  uint8_t* ch = P.xr + (static_cast<size_t>(ctile) * P.nb + sb) * kChunkBytes;
  uint32_t* pay = reinterpret_cast<uint32_t*>(ch + kChunkPay);
  float2* fac = reinterpret_cast<float2*>(ch + kChunkFac);
  __bf16* bmin = reinterpret_cast<__bf16*>(ch + kChunkMin);
  // every pass's load first (eight 16-byte loads in flight per thread)
  float4 vs[8];
#pragma unroll
  for (int ps = 0; ps < 8; ++ps) {
    const int b = ps * 32 + (threadIdx.x >> 3);
    const int s = b & 7, col = b >> 3;
    vs[ps] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (col < ncols)
      vs[ps] = *reinterpret_cast<const float4*>(P.xf + static_cast<size_t>(s_rows[col]) * kf +
                                                static_cast<size_t>(sb * 8 + s) * 32 + 4 * part);
  }
#pragma unroll
  for (int ps = 0; ps < 8; ++ps) {
    const int b = ps * 32 + (threadIdx.x >> 3);
    const int s = b & 7, col = b >> 3;
    const float4 v = vs[ps];
    uint32_t packed;
    float d;
    int S;
    q8_1_block_8lanes_vals(v, packed, d, S);
    pay[((2 * s + (part >> 2)) * 32 + col) * 4 + (part & 3)] = packed;
    if (part == 0) {
      const float beta = h2f(f2h_bits(d) & 0xffffu);  // the stored f16 scale
      fac[s * 32 + col] = make_float2(beta, -beta * kMagic);
      split3_bf16(beta * static_cast<float>(S), bmin[col * 8 + s], bmin[(32 + col) * 8 + s],
                  bmin[(64 + col) * 8 + s]);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void mmq_repack_kernel(RepackParams P) {
  const int sb = blockIdx.x, ctile = P.ct0 + static_cast<int>(blockIdx.y);
  const int s = threadIdx.x >> 5, col = threadIdx.x & 31;
  if (P.counters != nullptr && sb == 0 && ctile == 0) {
    if (threadIdx.x < kXcds) P.counters[threadIdx.x] = 0u;
    // 256 threads: every split-K arrival counter (dense calls only: a grouped
    // call's workspace holds its route tables there)
    if (MODE != kMoe) P.counters[kTileCntWord + threadIdx.x] = 0u;
    // grouped: also the queue of the down product of a fused FFN layer, whose
    // activation chunks the gate||up kernel writes (it has no repack of its own)
    if (MODE == kMoe && threadIdx.x < kXcds) P.counters[kXcds + threadIdx.x] = 0u;
  }
  __shared__ int s_ct[MODE == kMoe ? kMoeMaxE + 1 : 1];
  if constexpr (MODE == kMoe) {
    for (int i = threadIdx.x; i <= P.E; i += 256) s_ct[i] = P.ct_off[i];
    __syncthreads();
    if (ctile >= s_ct[P.E]) return;  // uniform: past the routed column tiles
  }
  if (MODE != kDebug && P.xf != nullptr) {  // uniform
    repack_f32<MODE>(P, s_ct, sb, ctile);
    return;
  }
  int xrow, ncols;
  if (!repack_row<MODE>(P, s_ct, ctile, col, xrow, ncols)) return;
  uint2 u[5];
  if (col < ncols) {
    const uint2* src = reinterpret_cast<const uint2*>(
        P.xq + static_cast<size_t>(xrow) * P.nb * 8 * kQ8Bytes + static_cast<size_t>(sb * 8 + s) * kQ8Bytes);
#pragma unroll
    for (int k = 0; k < 5; ++k) u[k] = src[k];
  } else {
#pragma unroll
    for (int k = 0; k < 5; ++k) u[k] = make_uint2(0u, 0u);
  }
  uint8_t* ch = P.xr + (static_cast<size_t>(ctile) * P.nb + sb) * kChunkBytes;
  uint4* pay = reinterpret_cast<uint4*>(ch + kChunkPay);
  pay[(2 * s) * 32 + col] = make_uint4(u[0].y, u[1].x, u[1].y, u[2].x);      // q[0..15]
  pay[(2 * s + 1) * 32 + col] = make_uint4(u[2].y, u[3].x, u[3].y, u[4].x);  // q[16..31]
  const float beta = h2f(u[0].x & 0xffffu);
  const int S = static_cast<int>(u[4].y);
  reinterpret_cast<float2*>(ch + kChunkFac)[s * 32 + col] = make_float2(beta, -beta * kMagic);
  __bf16* bmin = reinterpret_cast<__bf16*>(ch + kChunkMin);
  split3_bf16(beta * static_cast<float>(S), bmin[col * 8 + s], bmin[(32 + col) * 8 + s], bmin[(64 + col) * 8 + s]);
  // debug: the stored sums, Q4_K only (the Q6_K hook passes no S buffer)
  if (MODE == kDebug && P.dbgS != nullptr && col < ncols)
    P.dbgS[static_cast<size_t>(xrow) * P.nb * 8 + sb * 8 + s] = S;
}

// ----------------------------------------------------------------------------
// Main kernel
// ----------------------------------------------------------------------------
// How a step is split between the K halves (wave groups) of a workgroup.
// KS = 2 (the default): Q4_K: a step is two super-blocks; half kh takes
// super-block 2*step + kh (its 8 sub-blocks).  Q6_K: a step is one
// super-block; half kh takes its elements 128kh .. 128kh+127, i.e. MFMA
// sub-blocks 8kh .. 8kh+7 (half the weight bytes per wave, so the 64-column
// tile fits the register budget).  KS = 1 (Q4_K / Q5_K grouped calls): no K
// split, a step is one super-block taken by every wave for its own 32 rows,
// and the tile has 256 rows.  Either way a wave
// multiplies 8 MFMA sub-blocks per step.
template <int FMT, int KS = 2>
struct StepSplit {
  static_assert(KS == 2 || (KS == 1 && is_q4fam(FMT)), "K split");
  static constexpr int kSbPerStep = is_q4fam(FMT) ? KS : 1;
  static constexpr int kNU = 8;                        // MFMA sub-blocks per wave per step
  static constexpr int kSubsPerSb = is_q4fam(FMT) ? 8 : 16;
  static constexpr int kRowGroups = 8 / KS;            // 32-row groups per tile
  static constexpr int kBM = 32 * kRowGroups;          // weight rows per tile
  __device__ __forceinline__ static int sb(int step, int kh) { return is_q4fam(FMT) ? KS * step + kh : step; }
  __device__ __forceinline__ static int u0(int kh) { return is_q4fam(FMT) ? 0 : 8 * kh; }   // first sub-block
  __device__ __forceinline__ static int chunk_half(int kh) { return is_q4fam(FMT) ? kh : 0; }
  __host__ __device__ static int nsteps(int nb) { return is_q4fam(FMT) ? (nb + KS - 1) / KS : nb; }
};

template <int FMT, int NT, int KS = 2>
struct MmqSmem {
  static constexpr int kChunks = StepSplit<FMT, KS>::kSbPerStep * NT * kChunkBytes;  // [half][ct] chunks
  static constexpr int kRed = KS == 2 ? 4 * NT * 16 * 64 * 4 : 0;                    // K-half / split-K reduction
  static constexpr int kStage = kChunks > kRed ? kChunks : kRed;
  // alpha [8 sub-blocks][32 rows] fp32, then for Q4_K / Q5_K the min-term A
  // operand [3 parts][32 rows][8 sub-blocks] bf16
  static constexpr int kWave = 8 * 32 * 4 + (is_q4fam(FMT) ? 3 * 32 * 8 * 2 : 0);
  static constexpr int kWaveOff = 2 * kStage;
  static constexpr int kBytes = kWaveOff + kMmqWaves * kWave;
};

// Registers holding one super-block's weight bytes between their loads and
// their use (the software pipeline's in-flight stage).
template <int FMT>
struct MmqPrefetch;
template <>
struct MmqPrefetch<QMM_Q4_K> {
  uint4 hdr;   // d, dmin, packed scales
  uint4 q[4];  // bytes 16 + 32p + 16g .. +15: nibbles of sub-blocks 2p, 2p+1 for this lane's k-group
};
template <>
struct MmqPrefetch<QMM_Q5_K> {
  uint4 hdr;   // d, dmin, packed scales
  uint4 q[4];  // bytes 48 + 32p + 16g .. +15: nibbles of sub-blocks 2p, 2p+1 for this lane's k-group
  uint4 qh;    // bytes 16 + 16g .. +15: the fifth bits of the same 16 weights of every sub-block
};
template <>
struct MmqPrefetch<QMM_Q6_K> {
  // this wave's half of the super-block: per 16-group hf its qh bytes, per
  // (parity, hf) its ql bytes (8 bytes each as raw aligned dwords + shift),
  // the 4 scales this lane decodes (two 2-byte loads), d
  uint32_t qh_raw[2][3], ql_raw[2][2][3], sc_lo, sc_hi, d_raw, sh;
};

// 8 bytes at p (2-byte aligned) from three raw aligned dwords and the shift.
// The third dword is always read (no divergent branch): callers only use it
// for pieces that end at least 4 bytes before the end of their block.
__device__ __forceinline__ void raw8_load(const uint8_t* p, uint32_t (&r)[3], uint32_t& sh) {
  sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p - sh);  // stays a global pointer
  r[0] = base[0];
  r[1] = base[1];
  r[2] = base[2];
}
__device__ __forceinline__ uint2 raw8_join(const uint32_t (&r)[3], uint32_t sh) {
  return make_uint2(__builtin_amdgcn_alignbyte(r[1], r[0], sh), __builtin_amdgcn_alignbyte(r[2], r[1], sh));
}


// Weight bytes of super-block sb for this lane (row wr, k-group g), one
// load slot at a time.
//   Q4_K: slot 0 the header (d, dmin, packed scales), slots 1..4 the 16
//   value bytes 16 + 32p + 16g of pair p = u - 1.
//   Q6_K (half kh of the block): slots 0..5 the 8-byte pieces of 16-group hf:
//   qh, then ql of parity 0 and 1; slot 6 the 4 scales this lane decodes;
//   slot 7 d.
__device__ __forceinline__ void load_weight_slot(MmqPrefetch<QMM_Q4_K>& F, const uint8_t* wr, int sb, int g,
                                                 int u, int /*kh: whole block*/) {
  const uint8_t* blk = wr + static_cast<size_t>(sb) * kQ4Bytes;
  if (u == 0) F.hdr = ld16_a16(blk);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (u == p + 1) F.q[p] = ld16_a16(blk + 16 + 32 * p + 16 * g);
}
//   Q5_K: as Q4_K with the values at 48 + 32p + 16g; slot 5 the fifth bits
//   16 + 16g .. +15.
__device__ __forceinline__ void load_weight_slot(MmqPrefetch<QMM_Q5_K>& F, const uint8_t* wr, int sb, int g,
                                                 int u, int /*kh: whole block*/) {
  const uint8_t* blk = wr + static_cast<size_t>(sb) * kQ5Bytes;
  if (u == 0) F.hdr = ld16_a16(blk);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (u == p + 1) F.q[p] = ld16_a16(blk + 48 + 32 * p + 16 * g);
  if (u == 5) F.qh = ld16_a16(blk + 16 + 16 * g);
}
__device__ __forceinline__ void load_weight_slot(MmqPrefetch<QMM_Q6_K>& F, const uint8_t* wr, int sb, int g,
                                                 int u, int kh) {
  // half kh of the block: qh bytes 128 + 32kh + 16hf + 8g, ql bytes
  // 64kh + 32par + 16hf + 8g (each piece ends by byte 192, so the raw loads'
  // extra dword stays inside the 210-byte block), scales 192 + 8kh + 4g
  // (4 of them), d at 208
  const uint8_t* blk = wr + static_cast<size_t>(sb) * kQ6Bytes;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (u == 3 * hf) raw8_load(blk + 128 + 32 * kh + 16 * hf + 8 * g, F.qh_raw[hf], F.sh);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      if (u == 3 * hf + 1 + par) raw8_load(blk + 64 * kh + 32 * par + 16 * hf + 8 * g, F.ql_raw[par][hf], F.sh);
  }
  if (u == 6) {
    F.sc_lo = ld_u16(blk + 192 + 8 * kh + 4 * g);
    F.sc_hi = ld_u16(blk + 194 + 8 * kh + 4 * g);
  }
  if (u == 7) F.d_raw = ld_u16(blk + 208);
}

// A operand bytes of one super-block for this lane (row col of the wave's
// 32 rows, k-group g), taken out of the prefetch registers before the loads
// of the next super-block reuse them.
template <int FMT>
struct MmqOperand;
template <>
struct MmqOperand<QMM_Q4_K> {
  uint4 q[4];
};
template <>
struct MmqOperand<QMM_Q5_K> {
  uint4 q[4], qh;
};
template <>
struct MmqOperand<QMM_Q6_K> {
  uint2 ql[2][2], qh[2];  // this half's [parity][16-half] low-nibble bytes, [16-half] high-bit bytes
};

__device__ __forceinline__ void take_operand(const MmqPrefetch<QMM_Q4_K>& F, MmqOperand<QMM_Q4_K>& A) {
#pragma unroll
  for (int p = 0; p < 4; ++p) A.q[p] = F.q[p];
}
__device__ __forceinline__ void take_operand(const MmqPrefetch<QMM_Q5_K>& F, MmqOperand<QMM_Q5_K>& A) {
#pragma unroll
  for (int p = 0; p < 4; ++p) A.q[p] = F.q[p];
  A.qh = F.qh;
}
__device__ __forceinline__ void take_operand(const MmqPrefetch<QMM_Q6_K>& F, MmqOperand<QMM_Q6_K>& A) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    A.qh[hf] = raw8_join(F.qh_raw[hf], F.sh);
#pragma unroll
    for (int par = 0; par < 2; ++par) A.ql[par][hf] = raw8_join(F.ql_raw[par][hf], F.sh);
  }
}

// One column tile (NT = 1: MoE tiles, dense calls of up to 32 tokens): a
// lean register budget of 128 VGPRs, so four waves per SIMD (two workgroups
// per CU) share each SIMD and one workgroup's barriers and load waits are
// covered by the other's work, instead of the software pipelining over
// sub-blocks that the two-tile kernel uses.  To fit, a step's loads are all
// issued before its sub-block loop (no per-slot addresses kept live), one
// operand set and one MFMA result are live at a time, and the epilogue reads
// the row scales from LDS four at a time.
template <int FMT, int NT>
constexpr bool kLean = NT == 1;

// Decoded weight scales of this wave's rows to the wave's LDS region:
// alpha[u][row] = d*sc and, for Q4_K, mu[j][row] = -dmin*m.
template <int FMT>
__device__ __forceinline__ void write_scales_q4fam(const MmqPrefetch<FMT>& F, float* wave_lds, int col, int g) {
  // lane (row col, half g) decodes sub-blocks 4g .. 4g+3 of its row, whose
  // four 6-bit scales and mins come out as the bytes of one dword each (the
  // packing of q4k_scale_min, four sub-blocks at a time): sub-blocks 0-3
  // take bits 0-5 of S[0..3] (scales) and S[4..7] (mins); sub-blocks 4-7 the
  // nibbles of S[8..11] (low: scales, high: mins) with bits 6-7 of S[0..3]
  // (scales) and S[4..7] (mins) as bits 4-5
  const float d = h2f(F.hdr.x & 0xffffu), dmin = h2f(F.hdr.x >> 16);
  const uint32_t s0 = F.hdr.y, s1 = F.hdr.z, s2 = F.hdr.w;
  const uint32_t sc = g == 0 ? s0 & 0x3f3f3f3fu : (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u);
  const uint32_t mn = g == 0 ? s1 & 0x3f3f3f3fu : ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u);
  float* wa = wave_lds + 4 * g * 32 + col;
  // -dmin*m (exact in fp32: at most 17 significant bits) as three bf16 parts
  // by truncation: p0 keeps its top 8 significant bits, p1 the next 8 of the
  // exact remainder, p2 (at most one bit) the rest, so p0 + p1 + p2 = -dmin*m
  uint32_t part[3][4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    wa[jj * 32] = d * static_cast<float>((sc >> (8 * jj)) & 0xffu);
    const float x = -(dmin * static_cast<float>((mn >> (8 * jj)) & 0xffu));
    const uint32_t p0 = __float_as_uint(x) & 0xffff0000u;
    const float r = x - __uint_as_float(p0);
    const uint32_t p1 = __float_as_uint(r) & 0xffff0000u;
    part[0][jj] = p0;
    part[1][jj] = p1;
    part[2][jj] = __float_as_uint(r - __uint_as_float(p1));
  }
  // bf16 = the high half of each part; [3 parts][32 rows][8 sub-blocks]
  uint2* wm = reinterpret_cast<uint2*>(wave_lds + 8 * 32);
#pragma unroll
  for (int q = 0; q < 3; ++q)
    wm[(q * 32 + col) * 2 + g] = make_uint2((part[q][0] >> 16) | (part[q][1] & 0xffff0000u),
                                            (part[q][2] >> 16) | (part[q][3] & 0xffff0000u));
}
__device__ __forceinline__ void write_scales(const MmqPrefetch<QMM_Q4_K>& F, float* wave_lds, int col, int g) {
  write_scales_q4fam(F, wave_lds, col, g);
}
__device__ __forceinline__ void write_scales(const MmqPrefetch<QMM_Q5_K>& F, float* wave_lds, int col, int g) {
  write_scales_q4fam(F, wave_lds, col, g);
}
__device__ __forceinline__ void write_scales(const MmqPrefetch<QMM_Q6_K>& F, float* wave_lds, int col, int g) {
  // lane (row col, k-group g) holds scales 8kh + 4g .. +3 of its row: local sub-blocks 4g .. 4g+3
  const float d = h2f(F.d_raw);
  const uint32_t word = F.sc_lo | (F.sc_hi << 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wave_lds[(4 * g + q) * 32 + col] = d * static_cast<float>(static_cast<int8_t>((word >> (8 * q)) & 0xffu));
}

// Q4_K / Q5_K min term of a super-block: three bf16 MFMAs per column tile,
// MFMA k (issued after the epilogue of sub-block 2k + 1) taking the (A part,
// B part) products 2k and 2k + 1 in its two lane halves.  A[i][kk] = part of
// -dmin*m of row i (the wave's LDS region), B[kk][j] = part of beta*S of
// column j (the chunk), kk = 8 * half + sub-block.  Both kernel variants add
// it to each accumulator at the same point, so a product computed by the
// one- or the two-column-tile kernel has the same bits.
__device__ __forceinline__ bool min_slot(int u) { return u == 1 || u == 3 || u == 5; }

__device__ __forceinline__ v8bf min_a(const float* wl, int u) {
  const int g = (threadIdx.x & 63) >> 5, col = threadIdx.x & 31;
  return *reinterpret_cast<const v8bf*>(reinterpret_cast<const uint8_t*>(wl + 8 * 32) +
                                        (min_part_a(2 * (u >> 1) + g) * 32 + col) * 16);
}
__device__ __forceinline__ v8bf min_b(const uint8_t* chunk, int u) {
  const int g = (threadIdx.x & 63) >> 5, col = threadIdx.x & 31;
  return *reinterpret_cast<const v8bf*>(chunk + kChunkMin + (min_part_b(2 * (u >> 1) + g) * 32 + col) * 16);
}

// LDS operands of one MFMA sub-block u for this lane: the 16 row scales
// alpha of its rows, (beta, -beta*C) and the B operand of each column tile,
// and for Q4_K at odd u the min-term operands of sub-blocks u-1, u.
template <int FMT, int NT>
struct SubOps {
  using BQ = std::conditional_t<is_q4fam(FMT), v4i, long>;
  float al[16];
  float2 bp[NT];
  BQ bq[NT];
  v8bf am, bm[NT];   // min-term operands (two-tile kernel, Q4_K / Q5_K, min_slot(u))
};

// u indexes MFMA sub-blocks of the super-block: Q4_K u = the 32-weight
// sub-block (= Q8_1 block); Q6_K u = 2*s + hf, 16-weight group hf of Q8_1
// block s.  ul = u - (first sub-block of this wave's half) indexes the
// wave's scale region wl; st = this half's chunks ([ct] x kChunkBytes).
template <int FMT, int NT>
__device__ __forceinline__ void load_sub(const uint8_t* st, const float* wl, int u, int ul, SubOps<FMT, NT>& O) {
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  const int s = is_q4fam(FMT) ? u : u >> 1;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const uint8_t* ch = st + ct * kChunkBytes;
    if constexpr (is_q4fam(FMT))
      O.bq[ct] = *reinterpret_cast<const v4i*>(ch + kChunkPay + ((2 * s + g) * 32 + col) * 16);
    else
      O.bq[ct] = *reinterpret_cast<const long*>(ch + kChunkPay + ((2 * s + (u & 1)) * 32 + col) * 16 + 8 * g);
    O.bp[ct] = reinterpret_cast<const float2*>(ch + kChunkFac)[s * 32 + col];
  }
  if constexpr (is_q4fam(FMT)) {
    if (min_slot(u)) {
      O.am = min_a(wl, u);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) O.bm[ct] = min_b(st + ct * kChunkBytes, u);
    }
  }
  if constexpr (!kLean<FMT, NT>) {  // the lean epilogue reads them itself
    const float* wa = wl + ul * 32 + 4 * g;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 t4 = *reinterpret_cast<const float4*>(wa + 8 * k);
      O.al[4 * k] = t4.x; O.al[4 * k + 1] = t4.y; O.al[4 * k + 2] = t4.z; O.al[4 * k + 3] = t4.w;
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
//   Q5_K: as Q4_K with bit u of the fifth-bit bytes as bit 4 (0..31).
__device__ __forceinline__ v4i build_a(const MmqOperand<QMM_Q5_K>& A, int u) {
  const uint4 qv = A.q[u >> 1];
  const int sh = (u & 1) * 4;
  return v4i{static_cast<int>(((qv.x >> sh) & 0x0f0f0f0fu) | (((A.qh.x >> u) & 0x01010101u) << 4)),
             static_cast<int>(((qv.y >> sh) & 0x0f0f0f0fu) | (((A.qh.y >> u) & 0x01010101u) << 4)),
             static_cast<int>(((qv.z >> sh) & 0x0f0f0f0fu) | (((A.qh.z >> u) & 0x01010101u) << 4)),
             static_cast<int>(((qv.w >> sh) & 0x0f0f0f0fu) | (((A.qh.w >> u) & 0x01010101u) << 4))};
}
__device__ __forceinline__ long build_a(const MmqOperand<QMM_Q6_K>& A, int u) {
  // u in this wave's half: its half h is implied by the operand bytes taken
  const int s = u >> 1, hf = u & 1;
  const int gg = s & 3, par = gg & 1, shl = 4 * (gg >> 1), shh = 2 * gg;
  const uint2 lq = A.ql[par][hf];
  const uint2 hq = A.qh[hf];
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

// Token (output row) of column j of a tile, and whether it is valid.
struct TileCols {
  int n0, ncols;      // first column (dense) or first routed slot index (MoE), valid columns
  int slot_base;      // MoE: offset of the expert's slots in bucket
};

template <int MODE>
__device__ __forceinline__ int col_out_row(const MmqParams& P, const TileCols& tc, int j, bool& valid) {
  valid = j < tc.ncols;
  if constexpr (kIsMoe<MODE>) {
    return valid ? P.bucket[tc.slot_base + tc.n0 + j] : 0;
  } else {
    return tc.n0 + j;
  }
}

// Epilogue of (sub-block u of the step, column tile ct): acc += alpha *
// beta * D, and for Q4_K every second sub-block the min term.  Debug mode
// writes the integer sums D instead.
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void mmq_epilogue(const MmqParams& P, const TileCols& tc, int r0, int sb, int ub, int u,
                                             int ct, const v16i& Xc, const SubOps<FMT, NT>& Ou, v16f (&acc)[NT],
                                             const float* wl = nullptr, int ul = 0,
                                             const uint8_t* Xchunk = nullptr) {
  if constexpr (MODE == kDebug) {
    constexpr int NSB = StepSplit<FMT>::kSubsPerSb;
    const int g = (threadIdx.x & 63) >> 5, col = threadIdx.x & 31;
    bool ok;
    const int orr = col_out_row<MODE>(P, tc, ct * 32 + col, ok);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = r0 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (ok && row < P.M)
        P.dbgD[(static_cast<size_t>(orr) * P.M + row) * (P.nb * NSB) + sb * NSB + ub + u] =
            Xc[v] - static_cast<int>(kMagicBits);
    }
  } else {
    // the whole vector is reinterpreted: X holds 1.5*2^23 + D as fp32 bits
    const v16f Xf = __builtin_bit_cast(v16f, Xc);
    const float2 bp = Ou.bp[ct];
    if constexpr (kLean<FMT, NT>) {
      // row scales of sub-block ul from the wave's LDS region, four at a time
      const float* wa = wl + ul * 32 + 4 * ((threadIdx.x & 63) >> 5);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a4 = *reinterpret_cast<const float4*>(wa + 8 * k);
        const float al4[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float t = __builtin_fmaf(bp.x, Xf[4 * k + i], bp.y);
          acc[ct][4 * k + i] = __builtin_fmaf(al4[i], t, acc[ct][4 * k + i]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float t = __builtin_fmaf(bp.x, Xf[v], bp.y);
        acc[ct][v] = __builtin_fmaf(Ou.al[v], t, acc[ct][v]);
      }
    }
    if constexpr (is_q4fam(FMT)) {
      if (min_slot(u)) {
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ou.am, Ou.bm[ct], acc[ct], 0, 0, 0);
      }
    }
  }
}

template <int FMT, int NT, int KS>
struct StepLoads;

// Issue priority from the progress through a step's u of nu sub-blocks.
__device__ __forceinline__ void step_prio(int u, int nu) {
  const int q = (4 * u) / nu;
  if (q <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Multiply-accumulate this wave's 8 MFMA sub-blocks of a step (its rows, its
// half's chunks; ub = first sub-block of the half within the super-block).
// Software pipelined over sub-blocks so that the matrix core and the LDS
// reads run under the epilogue (see the two cases below).
template <int FMT, int NT, int MODE>
__device__ __forceinline__ void mmq_compute(const MmqParams& P, const uint8_t* st, const float* wl,
                                            const MmqOperand<FMT>& A, v16f (&acc)[NT], const v16i& magic,
                                            const TileCols& tc, int r0, int sb, int ub) {
  constexpr int NU = StepSplit<FMT>::kNU;  // MFMA sub-blocks of this wave per step
  if constexpr (kLean<FMT, NT>) {
    // one operand set and one result buffer per sub-block
    SubOps<FMT, NT> O;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      load_sub<FMT, NT>(st, wl, ub + u, u, O);
      const v16i X = mfma_sub(build_a(A, u), O.bq[0], magic);
      __builtin_amdgcn_sched_barrier(0);
      mmq_epilogue<FMT, NT, MODE>(P, tc, r0, sb, ub, u, 0, X, O, acc, wl, u, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // Two column tiles: the MFMA of (u+1, ct) is issued right after the
    // epilogue of (u, ct) has consumed its result registers, so it runs under
    // the epilogue of the next column tile; LDS operands of u+1 are read
    // while u is rescaled.  The two waves of a SIMD (the K halves of one row
    // group) share its issue slots and the arbiter favours the older one; the
    // issue priority falls as a wave gets through its step (3 in the first
    // quarter of its sub-blocks, 0 in the last), so the wave that is behind
    // is issued first and the pair reaches the step's barrier together.
    SubOps<FMT, NT> O[2];
    v16i X[NT];
    load_sub<FMT, NT>(st, wl, ub, 0, O[0]);
    {
      const auto a0 = build_a(A, 0);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) X[ct] = mfma_sub(a0, O[0].bq[ct], magic);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      step_prio(u, NU);
      const int b = u & 1;
      const bool more = u + 1 < NU;
      if (more) load_sub<FMT, NT>(st, wl, ub + u + 1, u + 1, O[b ^ 1]);
      const auto an = build_a(A, more ? u + 1 : u);
      // scheduling barriers pin the order: operand reads of u+1 first, then
      // per column tile its epilogue followed by its next MFMA
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        mmq_epilogue<FMT, NT, MODE>(P, tc, r0, sb, ub, u, ct, X[ct], O[b], acc, wl);
        if (more) X[ct] = mfma_sub(an, O[b ^ 1].bq[ct], magic);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Per-thread addressing of one tile.
struct TileRef {
  TileCols tc;
  int ctile0;             // first chunk row (column tile) of the tile
  int nct;                // valid column tiles (chunks) in the tile
  int r0;                 // first row of this wave
  const uint8_t* wr;      // weight row of this lane
  int s0, s1;             // steps of the tile's K range run here
  int base, split;        // dense split-K: tile and split index
};

// MoE tables copied to LDS at kernel start: the tile search runs in LDS
// instead of as a chain of dependent global loads.
struct MoeTables {
  const int* counts;    // [E]
  const int* offsets;   // [E]
  const int* ct_off;    // [E+1]
};

template <int FMT, int NT, int MODE, int KS>
__device__ __forceinline__ void tile_ref(const MmqParams& P, const MoeTables& Tb, int idx, TileRef& R) {
  using SP = StepSplit<FMT, KS>;
  constexpr int BN = 32 * NT;
  int m_tile;
  const uint8_t* wbase = P.w;
  if constexpr (kIsMoe<MODE>) {
    // expert e owns work entries [mt * ct_off[e], mt * ct_off[e + 1]): the
    // one with ct_off[e] <= idx / mt < ct_off[e + 1]
    const int q = idx / P.mt;
    int lo = 0, hi = P.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (Tb.ct_off[mid] <= q) lo = mid; else hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int cnt = __builtin_amdgcn_readfirstlane(Tb.counts[e]);
    const int ntile = (cnt + BN - 1) / BN;
    const int local = idx - P.mt * __builtin_amdgcn_readfirstlane(Tb.ct_off[e]);
    m_tile = local / ntile;
    const int n_tile = local % ntile;
    R.tc.n0 = n_tile * BN;
    R.tc.ncols = min(BN, cnt - R.tc.n0);
    R.tc.slot_base = Tb.offsets[e];
    R.ctile0 = Tb.ct_off[e] + n_tile * NT;
    wbase = P.w + static_cast<size_t>(e) * static_cast<size_t>(P.expert_stride);
  } else {
    const int ntile = (P.T + BN - 1) / BN;
    R.base = __builtin_amdgcn_readfirstlane(idx / P.nsplit);
    R.split = __builtin_amdgcn_readfirstlane(idx % P.nsplit);
    // tiles in runs of kGroupM row tiles x every column tile, row tile
    // fastest: the 32 workgroups of an XCD work on 8 row tiles x 4 column
    // tiles at a time, so their weight rows and activation chunks stay in
    // the XCD's L2 (column tile fastest had them sweep all the chunks)
    const int mtiles = (P.M + SP::kBM - 1) / SP::kBM;
    const int grp = R.base / (kGroupM * ntile), inner = R.base % (kGroupM * ntile);
    const int gm = min(kGroupM, mtiles - grp * kGroupM);
    m_tile = grp * kGroupM + inner % gm;
    const int n_tile = inner / gm;
    R.tc.n0 = n_tile * BN;
    R.tc.ncols = min(BN, P.T - R.tc.n0);
    R.tc.slot_base = 0;
    R.ctile0 = n_tile * NT;
  }
  // every value above is the same in all lanes (the tile index is): keep
  // them in scalar registers so the tile's control flow is scalar
  R.tc.n0 = __builtin_amdgcn_readfirstlane(R.tc.n0);
  R.tc.ncols = __builtin_amdgcn_readfirstlane(R.tc.ncols);
  R.tc.slot_base = __builtin_amdgcn_readfirstlane(R.tc.slot_base);
  R.ctile0 = __builtin_amdgcn_readfirstlane(R.ctile0);
  R.nct = (R.tc.ncols + kChunkCols - 1) / kChunkCols;
  m_tile = __builtin_amdgcn_readfirstlane(m_tile);
  {
    const int nsteps = SP::nsteps(P.nb);
    if constexpr (kIsMoe<MODE>) {
      R.s0 = 0;
      R.s1 = nsteps;
    } else {
      R.s0 = __builtin_amdgcn_readfirstlane(R.split * nsteps / P.nsplit);
      R.s1 = __builtin_amdgcn_readfirstlane((R.split + 1) * nsteps / P.nsplit);
    }
  }
  const int rw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % SP::kRowGroups;
  int wrow;
  if constexpr (MODE == kMoeGlu) {
    // wave rw: gate F-rows r0 .. r0 + 15 as MFMA rows 0..15, the matching
    // up rows (F-row + glu_f) as MFMA rows 16..31
    static_assert(SP::kRowGroups == 8, "the fused SwiGLU tile is 8 row groups");
    R.r0 = m_tile * 128 + rw * 16;
    const int i = threadIdx.x & 31;
    wrow = R.r0 + (i & 15) + (i >> 4) * P.glu_f;
  } else {
    R.r0 = m_tile * SP::kBM + rw * 32;
    wrow = min(R.r0 + (threadIdx.x & 31), P.M - 1);
  }
  constexpr int kRowBytes = FMT == QMM_Q4_K ? kQ4Bytes : FMT == QMM_Q5_K ? kQ5Bytes : kQ6Bytes;
  R.wr = wbase + static_cast<size_t>(wrow) * P.nb * kRowBytes;
}

// The loads of one step -- the chunks of its super-blocks (copied into LDS
// stage dst, [half][ct] chunks) and this wave's weight bytes -- all issued at
// the top of the previous step's compute.  Chunk copies: each wave
// instruction moves 1 KB (lane l the 16 bytes at 16*l); the step's kInstr
// copies are split into runs of kDma consecutive ones, run w for wave w, so
// that a wave's copies lie in one chunk: their addresses are one base plus
// multiples of 1 KB, the base fixed per wave (DmaPlan) plus a per-step term.
template <int FMT, int NT, int KS>
struct StepLoads {
  using SP = StepSplit<FMT, KS>;
  static constexpr int kInstr = SP::kSbPerStep * NT * kChunkKB;
  static constexpr int kDma = (kInstr + kMmqWaves - 1) / kMmqWaves;  // chunk copies per wave
  static_assert(kChunkKB % kDma == 0, "a wave's chunk copies must stay inside one chunk");
  static constexpr int kW = FMT == QMM_Q4_K ? 5 : FMT == QMM_Q5_K ? 6 : 8;  // weight loads per wave
  const uint8_t* src;      // this lane's 16 bytes of the wave's first copy
  uint32_t dst;            // LDS address of the wave's first copy
  bool dma;                // the wave copies in this step
  const uint8_t* wr;       // this lane's weight row of the loaded tile
  int sbw;                 // super-block of the wave's weight loads (< 0: none)
  int kh, g;

  __device__ __forceinline__ void issue_all(MmqPrefetch<FMT>& F) const {
    if (dma) {
#pragma unroll
      for (int i = 0; i < kDma; ++i) dma16(src + i * 1024, dst + i * 1024);
    }
    if (sbw >= 0) {
#pragma unroll
      for (int w = 0; w < kW; ++w) load_weight_slot(F, wr, sbw, g, w, kh);
    }
  }
};

// The part of a wave's chunk copies that does not change with the tile or the
// step: which chunk (half hj, column tile ct) and which 1 KB slice q0 of it
// its run starts at, as global and LDS offsets.
struct DmaPlan {
  size_t src_off;   // ((ct * nb) + hj) * kChunkBytes + q0 * 1 KB + 16 * lane
  uint32_t dst_off; // (hj * NT + ct) * kChunkBytes + q0 * 1 KB
  int hj, ct;
  bool has;         // the wave has a run
};

template <int FMT, int NT, int KS>
__device__ __forceinline__ DmaPlan dma_plan(int wave, int nb) {
  using L = StepLoads<FMT, NT, KS>;
  DmaPlan D;
  const int first = wave * L::kDma;
  D.has = first < L::kInstr;
  const int pair = first / kChunkKB, q0 = first % kChunkKB;
  D.hj = pair / NT;
  D.ct = pair % NT;
  D.src_off = (static_cast<size_t>(D.ct) * nb + D.hj) * kChunkBytes + q0 * 1024 + (threadIdx.x & 63) * 16;
  D.dst_off = static_cast<uint32_t>((D.hj * NT + D.ct) * kChunkBytes + q0 * 1024);
  return D;
}

template <int FMT, int NT, int KS>
__device__ __forceinline__ StepLoads<FMT, NT, KS> step_loads(const MmqParams& P, const TileRef& R,
                                                             const DmaPlan& D, int step, uint32_t dst, bool any,
                                                             int kh, int g) {
  using SP = StepSplit<FMT, KS>;
  StepLoads<FMT, NT, KS> L;
  const int sb0 = SP::kSbPerStep * step;
  L.src = P.xr + (static_cast<size_t>(R.ctile0) * P.nb + sb0) * kChunkBytes + D.src_off;
  L.dst = dst + D.dst_off;
  L.dma = any && D.has && D.ct < R.nct && sb0 + D.hj < P.nb;
  L.wr = R.wr;
  const int sbw = SP::sb(step, kh);
  L.sbw = any && sbw < P.nb ? sbw : -1;
  L.kh = kh;
  L.g = g;
  return L;
}

// Store a wave's 32 x (32*NT) fp32 tile.  acc[ct][v] holds row
// 8*(v/4) + 4*(lane/32) + v%4 of the wave's rows and column ct*32 + lane%32.
template <int NT, int MODE>
__device__ __forceinline__ void store_tile(const MmqParams& P, const TileCols& tc, int r0,
                                           const v16f (&acc)[NT]) {
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    bool valid;
    const int orow = col_out_row<MODE>(P, tc, ct * 32 + col, valid);
    if (!valid) continue;
    float* yr = P.y + static_cast<size_t>(orow) * P.M;
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

// Fused SwiGLU epilogue of a grouped gate||up tile (all waves call it).
// Wave w's 32 MFMA rows are 16 gate rows, F-rows r0 .. r0 + 15, then the 16
// matching up rows (tile_ref), so lane (col, g) holds gate row 8k + 4g + j in
// acc[4k + j] and its up row in acc[4(k + 2) + j] (k = 0, 1): h = silu(gate) *
// up is lane-local.  A Q8_1 block (32 F-rows of output row `slot`) spans the
// wave pair 2b, 2b + 1; its max |h| and integer sum are combined through LDS
// (the stage the tile last computed from, free after a barrier).  The steps
// are those of swiglu_q8_1, so the bytes are too.
template <int NT>
__device__ __forceinline__ void glu_store(const MmqParams& P, const TileRef& R, const v16f (&acc)[NT], int wave,
                                          int lane, uint8_t* stage) {
#pragma clang fp contract(off)
  const int g = lane >> 5, col = lane & 31;
  float h[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) h[v] = silu_mul(acc[0][v], acc[0][v + 8]);
  float am = 0.0f;
#pragma unroll
  for (int v = 0; v < 8; ++v) am = fmaxf(am, fabsf(h[v]));
  am = fmaxf(am, __shfl_xor(am, 32));
  float* xa = reinterpret_cast<float*>(stage);        // [8 waves][32 columns] max |h|
  int* xs = reinterpret_cast<int*>(stage + 1024);     // [8 waves][32 columns] sums
  __syncthreads();  // every wave is done with the stage
  if (g == 0) xa[wave * 32 + col] = am;
  __syncthreads();
  am = fmaxf(am, xa[(wave ^ 1) * 32 + col]);
  const float d = am / 127.0f;
  const float di = d >= 0x1p-126f ? 1.0f / d : 0.0f;
  int s = 0;
  uint32_t packed[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t pk = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = max(-128, min(127, static_cast<int>(rintf(h[4 * k + j] * di))));
      s += q;
      pk |= (static_cast<uint32_t>(q) & 255u) << (8 * j);
    }
    packed[k] = pk;
  }
  s += __shfl_xor(s, 32);
  if (g == 0) xs[wave * 32 + col] = s;
  __syncthreads();
  s += xs[(wave ^ 1) * 32 + col];
  if (P.xr_next != nullptr) {
    // the down product's chunk (column tile ctile0, super-block blk / 8),
    // sub-block s = blk % 8, as the routed-row repack lays it out: values of
    // half w % 2 at bytes 8k + 4g of entry (2s + w % 2, col), (beta, -beta*C),
    // the bf16 parts of beta*S.  Padded columns come out zero (their gate||up
    // sums are zero), as the repack writes them.
    const int blk = R.r0 / 32, sub = blk & 7;
    uint8_t* ch = P.xr_next + (static_cast<size_t>(R.ctile0) * P.nb_next + (blk >> 3)) * kChunkBytes;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      reinterpret_cast<uint32_t*>(ch + kChunkPay + ((2 * sub + (wave & 1)) * 32 + col) * 16 + 8 * k + 4 * g)[0] =
          packed[k];
    if ((wave & 1) == 0 && g == 0) {
      const float beta = h2f(f2h_bits(d) & 0xffffu);  // the stored f16 scale
      reinterpret_cast<float2*>(ch + kChunkFac)[sub * 32 + col] = make_float2(beta, -beta * kMagic);
      __bf16* bmin = reinterpret_cast<__bf16*>(ch + kChunkMin);
      split3_bf16(beta * static_cast<float>(s), bmin[col * 8 + sub], bmin[(32 + col) * 8 + sub],
                  bmin[(64 + col) * 8 + sub]);
    }
    return;
  }
  bool valid;
  const int orow = col_out_row<kMoeGlu>(P, R.tc, col, valid);
  if (valid) {
    // block r0 / 32 along F; this wave's F-rows sit at 16 (w % 2) .. + 15 in it
    uint8_t* dst = P.yq + (static_cast<size_t>(orow) * (P.glu_f / 32) + R.r0 / 32) * kQ8Bytes;
#pragma unroll
    for (int k = 0; k < 2; ++k) reinterpret_cast<uint32_t*>(dst + 4 + 16 * (wave & 1) + 8 * k + 4 * g)[0] = packed[k];
    if ((wave & 1) == 0 && g == 0) {
      reinterpret_cast<uint32_t*>(dst)[0] = f2h_bits(d);  // f16 d, zero pad
      reinterpret_cast<int32_t*>(dst + 36)[0] = s;
    }
  }
}

// Split-K epilogue of a dense tile (all waves call it; the kh == 0 waves
// hold the tile's partial sums).  The partial goes to the tile's slot in the
// workspace; after a barrier, thread 0 releases the workgroup's stores at
// device scope and bumps the tile's arrival counter.  The workgroup that
// arrives last acquires the other splits' stores and adds the nsplit
// partials in split order (its own from registers), so the sum does not
// depend on which split finishes last.
template <int NT, int MODE>
__device__ __forceinline__ void split_store(const MmqParams& P, const TileRef& R, const v16f (&acc)[NT], int rw,
                                            int lane, int kh, int& s_last) {
  constexpr size_t kTile = static_cast<size_t>(4) * NT * 16 * 64;  // floats per partial tile
  if (kh == 0) {
    float* mine = P.part + (static_cast<size_t>(R.base) * P.nsplit + R.split) * kTile;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) mine[((rw * NT + ct) * 16 + v) * 64 + lane] = acc[ct][v];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned old = atomicAdd(&P.tile_cnt[R.base], 1u);
    s_last = old + 1 == static_cast<unsigned>(P.nsplit);
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(s_last)) {
    __threadfence();
    if (kh == 0) {
      v16f sum[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum[ct][v] = 0.0f;
      for (int sp = 0; sp < P.nsplit; ++sp) {
        const float* ps = P.part + (static_cast<size_t>(R.base) * P.nsplit + sp) * kTile;
        const bool own = sp == R.split;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) sum[ct][v] += own ? acc[ct][v] : ps[((rw * NT + ct) * 16 + v) * 64 + lane];
      }
      store_tile<NT, MODE>(P, R.tc, R.r0, sum);
    }
  }
}

// Work queues.  The tiles are split into kXcds contiguous ranges, one per
// XCD (workgroup b runs on XCD b % kXcds), so a range's weight rows stay in
// one XCD's L2.  Workgroup b takes tile b / kXcds of its range as its first
// tile (no atomic on the critical path at start-up); every further tile
// comes from the range's atomic counter: ticket c is tile nw + c of the range,
// nw being the number of workgroups on that XCD.  A failed claim ends the
// workgroup.  The counters are zeroed by the kernel that runs before this one
// on the stream (activation repack or route preparation).
struct Queue {
  int start, size;  // tile range of this workgroup's XCD
  int nw;           // workgroups on this XCD
  int home;
};

__device__ __forceinline__ Queue make_queue(int total) {
  Queue Q;
  Q.home = static_cast<int>(blockIdx.x % kXcds);
  Q.start = static_cast<int>((static_cast<int64_t>(total) * Q.home) / kXcds);
  Q.size = static_cast<int>((static_cast<int64_t>(total) * (Q.home + 1)) / kXcds) - Q.start;
  Q.nw = static_cast<int>((gridDim.x - Q.home + kXcds - 1) / kXcds);
  return Q;
}

__device__ __forceinline__ void wait_vm_all() { wait_vmcnt<0>(); }

// Persistent loop over the tiles of the call.  Steps of two super-blocks
// (one per K half); at the top of a step every wave waits for its own loads
// of the step (issued during the previous step), then one barrier publishes
// the copied chunks and frees the other LDS stage, into which the next step's
// chunks are copied, slot by slot, while this step is computed.  Loads of a
// tile's first step are issued during the previous tile's last step.  The
// next tile is claimed one ahead: thread 0 issues the atomic at the top of a
// tile's first step and reads its value at the top of the tile's last step
// (after the full wait there, so with two or more steps it costs no stall),
// then publishes it before that step's barrier.
template <int FMT, int NT, int MODE, int KS = 2>
__global__ __launch_bounds__(kMmqThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 4 : 2, NT == 1 ? 4 : 2))) void mmq_kernel(MmqParams P) {
  using L = MmqSmem<FMT, NT, KS>;
  using SP = StepSplit<FMT, KS>;
  static_assert(KS == 2 || kIsMoe<MODE>, "the dense and debug calls split K in two");
  static_assert(MODE != kMoeGlu || (KS == 1 && NT == 1), "the fused SwiGLU runs on whole-K one-tile tiles");
  constexpr int kTab = kIsMoe<MODE> ? kMoeMaxE + 1 : 1;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  __shared__ int s_next[2];
  __shared__ int s_last;
  __shared__ int s_counts[kTab], s_offsets[kTab], s_ct_off[kTab];

  MoeTables Tb{s_counts, s_offsets, s_ct_off};
  int total;
  if constexpr (kIsMoe<MODE>) {
    for (int i = threadIdx.x; i <= P.E; i += kMmqThreads) {
      s_ct_off[i] = P.ct_off[i];
      if (i < P.E) {
        s_counts[i] = P.counts[i];
        s_offsets[i] = P.offsets[i];
      }
    }
    total = P.mt * __builtin_amdgcn_readfirstlane(P.ct_off[P.E]);
    __syncthreads();
  } else {
    total = ((P.M + kMmqBM - 1) / kMmqBM) * ((P.T + 32 * NT - 1) / (32 * NT)) * P.nsplit;
  }
  const Queue Q = make_queue(total);
  const int b8 = static_cast<int>(blockIdx.x / kXcds);
  if (b8 >= Q.size) return;  // no tile for this workgroup (uniform)
  const int lane = threadIdx.x & 63, g = lane >> 5, col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = KS == 2 ? wave >> 2 : 0;
  // The two waves of a SIMD (K halves 0 and 1) share its issue slots; the
  // arbiter favours the older one, so the second half used to finish each
  // step alone, its matrix-core latency exposed.  The two-tile kernel sets
  // the priority by progress through each step (see mmq_compute); the
  // one-tile Q6_K kernel raises the second half's priority instead.
  if (kLean<FMT, NT> && FMT == QMM_Q6_K && kh == 1) __builtin_amdgcn_s_setprio(2);
  float* wl = reinterpret_cast<float*>(smem + L::kWaveOff + wave * L::kWave);
  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = static_cast<int>(kMagicBits);
  // opaque to the compiler, so it stays in registers instead of being
  // rebuilt (16 moves) in front of every MFMA
  __asm__ volatile("" : "+v"(magic));
  TileRef R, Rn;
  tile_ref<FMT, NT, MODE, KS>(P, Tb, Q.start + b8, R);
  MmqPrefetch<FMT> F;
  const uint32_t lds0 = lds_addr(smem);
  const DmaPlan D = dma_plan<FMT, NT, KS>(wave, P.nb);
  {
    const StepLoads<FMT, NT, KS> first = step_loads<FMT, NT, KS>(P, R, D, R.s0, lds0, true, kh, g);
    first.issue_all(F);
  }
  int k = 0;            // steps done by this workgroup (selects the LDS stage)
  unsigned ticket = 0;  // thread 0: counter value of the claim of the next tile
  for (int it = 0;; ++it) {
    v16f acc[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ct][v] = 0.0f;
    int next = -1;
    for (int step = R.s0; step < R.s1; ++step, ++k) {
      uint8_t* st = smem + (k & 1) * L::kStage;
      const int sb = SP::sb(step, kh);
      const bool active = sb < P.nb;
      const bool last = step + 1 == R.s1;
      MmqOperand<FMT> A;
      if (active) {
        take_operand(F, A);
        write_scales(F, wl, col, g);
      }
      wait_vm_all();
      if (threadIdx.x == 0) {
        if (step == R.s0) ticket = atomicAdd(&P.counters[Q.home], 1u);
        if (last) {
          const int j = Q.nw + static_cast<int>(ticket);
          s_next[it & 1] = j < Q.size ? Q.start + j : -1;
        }
      }
      __syncthreads();
      if (last) {
        next = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
        if (next >= 0) tile_ref<FMT, NT, MODE, KS>(P, Tb, next, Rn);
      }
      const uint32_t dst = lds0 + ((k + 1) & 1) * L::kStage;
      const StepLoads<FMT, NT, KS> pre = last ? step_loads<FMT, NT, KS>(P, Rn, D, Rn.s0, dst, next >= 0, kh, g)
                                              : step_loads<FMT, NT, KS>(P, R, D, step + 1, dst, true, kh, g);
      pre.issue_all(F);
      if (active) {
        mmq_compute<FMT, NT, MODE>(P, st + SP::chunk_half(kh) * NT * kChunkBytes, wl, A, acc, magic, R.tc, R.r0,
                                   sb, SP::u0(kh));
      }
    }
    if constexpr (MODE == kMoeGlu) {
      glu_store<NT>(P, R, acc, wave, lane, smem + ((k - 1) & 1) * L::kStage);
    } else if constexpr (MODE != kDebug && KS == 1) {
      store_tile<NT, MODE>(P, R.tc, R.r0, acc);  // every wave holds whole sums of its 32 rows
    } else if constexpr (MODE != kDebug) {
      // sum the two K halves through the stage just computed from
      __syncthreads();
      float* red = reinterpret_cast<float*>(smem + ((k - 1) & 1) * L::kStage);
      const int rw = wave & 3;
      if (kh == 1) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) red[((rw * NT + ct) * 16 + v) * 64 + lane] = acc[ct][v];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[ct][v] += red[((rw * NT + ct) * 16 + v) * 64 + lane];
      }
      if (MODE == kDense && P.nsplit > 1) {
        split_store<NT, MODE>(P, R, acc, rw, lane, kh, s_last);
      } else if (kh == 0) {
        store_tile<NT, MODE>(P, R.tc, R.r0, acc);
      }
    }
    if (next < 0) break;
    R = Rn;
  }
}

// Grid size: per_cu workgroups per CU (eight waves each: two per SIMD, or
// four per SIMD for the lean one-tile kernel at two per CU), a multiple of
// the XCD count so every XCD range has workers.
static int mmq_grid(int total_tiles_hint, int per_cu) {
  int g = device_cu_count() * per_cu;
  if (total_tiles_hint > 0 && total_tiles_hint < g) g = total_tiles_hint;
  g = ((g + kXcds - 1) / kXcds) * kXcds;
  return g < kXcds ? kXcds : g;
}

template <int FMT, int NT, int MODE, int KS = 2>
static int launch_mmq(const MmqParams& P, int total_tiles_hint, hipStream_t st) {
  using L = MmqSmem<FMT, NT, KS>;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmq_kernel<FMT, NT, MODE, KS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const int grid = mmq_grid(total_tiles_hint, kLean<FMT, NT> ? 2 : 1);
  hipLaunchKernelGGL((mmq_kernel<FMT, NT, MODE, KS>), dim3(grid), dim3(kMmqThreads), L::kBytes, st, P);
  return launch_status();
}

// The repack grid is (super-blocks, column tiles); column tiles are launched
// in chunks of at most kMaxGridY along grid y (tens of thousands of column
// tiles for calls with millions of tokens or routed slots).
constexpr int kMaxGridY = 65535;

template <int MODE>
static int launch_repack(RepackParams R, int nb, int ctiles, hipStream_t st) {
  for (int c0 = 0; c0 < ctiles; c0 += kMaxGridY) {
    R.ct0 = c0;
    const int n = ctiles - c0 < kMaxGridY ? ctiles - c0 : kMaxGridY;
    hipLaunchKernelGGL(mmq_repack_kernel<MODE>, dim3(nb, n), dim3(256), 0, st, R);
    const int rc = launch_status();
    if (rc != QMM_OK) return rc;
  }
  return QMM_OK;
}

static size_t mmq_chunk_bytes(int64_t ctiles, int64_t nb) {
  return static_cast<size_t>(ctiles) * static_cast<size_t>(nb) * kChunkBytes;
}

// Column tiles per dense tile: two (64 tokens) for calls with more than 32
// tokens, else one.
static int mmq_dense_nt(int64_t T) { return T > 32 ? 2 : 1; }

// Dense tiles of a call (without split) and its split-K factor.
static int64_t mmq_dense_tiles(int64_t M, int64_t T) {
  const int64_t bn = 32 * mmq_dense_nt(T);
  return ((M + kMmqBM - 1) / kMmqBM) * ((T + bn - 1) / bn);
}
static int mmq_nsplit(int64_t M, int64_t K, int64_t T) {
  const int64_t tiles = mmq_dense_tiles(M, T);
  if (tiles >= kSplitTiles) return 1;
  int64_t n = kSplitTiles / tiles;
  const int64_t by_k = (K / kQK) / 4;  // at least four super-blocks per split
  if (n > by_k) n = by_k;
  if (n > kMaxSplit) n = kMaxSplit;
  return n < 1 ? 1 : static_cast<int>(n);
}
static size_t mmq_part_bytes(int64_t M, int64_t K, int64_t T) {
  const int ns = mmq_nsplit(M, K, T);
  if (ns == 1) return 0;
  return static_cast<size_t>(mmq_dense_tiles(M, T)) * ns * mmq_dense_nt(T) * 4 * 16 * 64 * sizeof(float);
}
static size_t mmq_part_offset(int64_t K, int64_t T) {
  const int64_t ctiles = (T + kChunkCols - 1) / kChunkCols;
  return (kCounterBytes + mmq_chunk_bytes(ctiles, K / kQK) + 255) / 256 * 256;
}

size_t mmq_workspace_bytes(int64_t M, int64_t K, int64_t T) {
  return mmq_part_offset(K, T) + mmq_part_bytes(M, K, T);
}

// Upper bound of the column tiles of a grouped call: sum over experts of
// ceil(count / 32) <= (slots + 31 * n) / 32 with n = min(E, slots) the most
// experts that can receive a slot.
int64_t moe_max_ctiles(int64_t slots, int64_t E) {
  const int64_t n = E < slots ? E : slots;
  return (slots + 31 * n) / 32;
}
size_t moe_chunk_bytes(int64_t slots, int64_t E, int64_t K) {
  return mmq_chunk_bytes(moe_max_ctiles(slots, E), K / kQK);
}

// Dense tiles are 128 rows x 64 tokens (128 x 32 for calls with few tokens).
template <int FMT>
static int mmq_dense_fmt(const MmqParams& P, bool dbg, hipStream_t st) {
  const int tiles = static_cast<int>(mmq_dense_tiles(P.M, P.T)) * P.nsplit;
  if (mmq_dense_nt(P.T) == 2)
    return dbg ? launch_mmq<FMT, 2, kDebug>(P, tiles, st) : launch_mmq<FMT, 2, kDense>(P, tiles, st);
  return dbg ? launch_mmq<FMT, 1, kDebug>(P, tiles, st) : launch_mmq<FMT, 1, kDense>(P, tiles, st);
}

int mmq_dense(int fmt, const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
              void* ws, hipStream_t st, int32_t* dbgD, int32_t* dbgS, const float* xf) {
  const bool dbg = dbgD != nullptr;
  uint8_t* xr = static_cast<uint8_t*>(ws) + kCounterBytes;
  const int nb = static_cast<int>(K / kQK);
  const int ctiles = static_cast<int>((T + kChunkCols - 1) / kChunkCols);
  RepackParams R{};
  R.xq = static_cast<const uint8_t*>(xq);
  R.xf = xf;
  R.xr = xr;
  R.nb = nb;
  R.T = static_cast<int>(T);
  R.dbgS = dbgS;
  R.counters = static_cast<unsigned*>(ws);
  int rc = dbg ? launch_repack<kDebug>(R, nb, ctiles, st) : launch_repack<kDense>(R, nb, ctiles, st);
  if (rc != QMM_OK) return rc;
  MmqParams P{};
  P.w = static_cast<const uint8_t*>(w);
  P.xr = xr;
  P.y = y;
  P.M = static_cast<int>(M);
  P.nb = nb;
  P.T = static_cast<int>(T);
  P.counters = static_cast<unsigned*>(ws);
  P.tile_cnt = static_cast<unsigned*>(ws) + kTileCntWord;
  P.nsplit = dbg ? 1 : mmq_nsplit(M, K, T);  // the integer-stage debug path writes per sub-block sums
  P.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + mmq_part_offset(K, T));
  P.dbgD = dbgD;
  if (fmt == QMM_Q4_K) return mmq_dense_fmt<QMM_Q4_K>(P, dbg, st);
  if (fmt == QMM_Q5_K) return mmq_dense_fmt<QMM_Q5_K>(P, dbg, st);
  return mmq_dense_fmt<QMM_Q6_K>(P, dbg, st);
}

// Weight rows per tile of a grouped call: 256 for Q4_K / Q5_K, every wave
// taking every super-block of its own 32 rows (no K halves: no idle half on
// the last step of rows with an odd number of super-blocks, no reduction of
// the halves per tile; the grouped FFN calls measured 4-8 % faster than with
// 128-row tiles split in K), 128 for Q6_K (its K halves split each
// super-block, so they never go idle).
int moe_tile_rows(int fmt, int /*nb*/) {
  return is_q4fam(fmt) ? StepSplit<QMM_Q4_K, 1>::kBM : StepSplit<QMM_Q6_K, 2>::kBM;
}

// Grouped launch used by moe_grouped_mmq (after route preparation on the
// same stream): repack of the routed rows per expert, then tiles of
// moe_tile_rows rows x 32 routed slots.
// hq != nullptr: the gate||up product (M = 2F rows) with SwiGLU -> Q8_1
// fused into the epilogue, Q8_1 rows of F / 32 blocks into hq (Q4_K / Q5_K,
// F % 128 == 0) instead of fp32 rows into out.
// xr_next != nullptr (with hq): the fused FFN layer's gate||up call, writing
// the down product's chunks (nb_next super-blocks) there instead of Q8_1 rows.
// repack == false: the chunks in xr were written that way; the GEMM runs on
// them with its queue counters at words 8.. (zeroed by the first repack).
int mmq_moe_launch(int fmt, const uint8_t* w, int64_t stride, int M, int nb, const uint8_t* xq,
                   float* out, uint8_t* hq, unsigned* counters, const int32_t* counts, const int32_t* offsets,
                   const int32_t* bucket, const int32_t* ct_off, uint8_t* xr,
                   int max_ctiles, int E, int top_k, int rows_per_token, hipStream_t st,
                   uint8_t* xr_next, int nb_next, bool repack) {
  RepackParams R{};
  R.xq = xq;
  R.xr = xr;
  R.nb = nb;
  R.counts = counts;
  R.offsets = offsets;
  R.bucket = bucket;
  R.ct_off = ct_off;
  R.E = E;
  R.top_k = top_k;
  R.rows_per_token = rows_per_token;
  R.counters = counters;  // zeroed for the GEMM (route tables reused from an earlier call leave them dirty)
  if (repack) {
    const int rc = launch_repack<kMoe>(R, nb, max_ctiles, st);
    if (rc != QMM_OK) return rc;
  } else {
    counters += kXcds;
  }
  MmqParams P{};
  P.w = w;
  P.xr = xr;
  P.y = out;
  P.M = M;
  P.nb = nb;
  P.T = 0;
  P.nsplit = 1;
  P.counters = counters;
  P.counts = counts;
  P.offsets = offsets;
  P.bucket = bucket;
  P.ct_off = ct_off;
  P.E = E;
  P.expert_stride = stride;
  const int bm = moe_tile_rows(fmt, nb);
  P.mt = (M + bm - 1) / bm;
  const bool whole_k = bm == StepSplit<QMM_Q4_K, 1>::kBM;
  if (hq != nullptr) {
    if (!whole_k || (M % 256) != 0) return QMM_ERR_UNSUPPORTED;
    P.yq = hq;
    P.xr_next = xr_next;
    P.nb_next = nb_next;
    P.glu_f = M / 2;
    P.mt = P.glu_f / 128;
    if (fmt == QMM_Q4_K) return launch_mmq<QMM_Q4_K, 1, kMoeGlu, 1>(P, 0, st);
    return launch_mmq<QMM_Q5_K, 1, kMoeGlu, 1>(P, 0, st);
  }
  if (fmt == QMM_Q4_K)
    return whole_k ? launch_mmq<QMM_Q4_K, 1, kMoe, 1>(P, 0, st) : launch_mmq<QMM_Q4_K, 1, kMoe>(P, 0, st);
  if (fmt == QMM_Q5_K)
    return whole_k ? launch_mmq<QMM_Q5_K, 1, kMoe, 1>(P, 0, st) : launch_mmq<QMM_Q5_K, 1, kMoe>(P, 0, st);
  return launch_mmq<QMM_Q6_K, 1, kMoe>(P, 0, st);
}

// Host checks of a GEMM call's sizes and operand pointers, then of its workspace.
static int check_mmq_args(const void* w, const void* xq, const float* y, int64_t M, int64_t K, int64_t T) {
  if (M < 1 || T < 1 || K < kQK || (K % kQK) != 0) return QMM_ERR_SHAPE;
  if (M > (1 << 30) || T > (1 << 24) || K / kQK > (1 << 16)) return QMM_ERR_SHAPE;
  // tile indices are 32-bit in the kernel
  if (mmq_dense_tiles(M, T) * mmq_nsplit(M, K, T) > (int64_t{1} << 30)) return QMM_ERR_SHAPE;
  if (!w || !xq || !y) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(y)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

static int check_mmq(const void* w, const void* xq, const float* y, int64_t M, int64_t K, int64_t T,
                     const void* ws, size_t ws_bytes) {
  const int st = check_mmq_args(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  if (!ws) return QMM_ERR_NULL;
  if (!aligned16(ws)) return QMM_ERR_ALIGN;
  if (ws_bytes < mmq_workspace_bytes(M, K, T)) return QMM_ERR_WORKSPACE;
  return QMM_OK;
}

// Scratch of mmq_q4k_noalloc: a device array of fixed size in the library's
// code object (each GPU the library runs on holds its own copy until the
// process ends), used instead of a caller workspace.  Host code never passes
// `scratch` itself to a kernel (on the host the name is only a stand-in for
// the symbol); it takes the array's device address, once per device, from
// hipGetSymbolAddress and passes that.
static __device__ __align__(256) uint8_t scratch[QMM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of this device's `scratch`, looked up on the device's first
// call (with the device current) and kept.
static int static_scratch(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QMM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QMM_ERR_HIP;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return QMM_OK;
}

}  // namespace qmm

using namespace qmm;

extern "C" int mmq_q4k_noalloc(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                               void* stream) {
  // the checks of mmq_q4k, with the static array in place of ws
  const int st = check_mmq_args(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  if (mmq_workspace_bytes(M, K, T) > QMM_STATIC_SCRATCH_BYTES) return QMM_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = static_scratch(&ws);
  if (rc != QMM_OK) return rc;
  // the activation repack that runs first zeroes the queue and split-K
  // counters in the scratch, so no clearing is needed here
  return mmq_dense(QMM_Q4_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, nullptr);
}

extern "C" int mmq_q4k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                       void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, xq, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q4_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, nullptr);
}

extern "C" int mmq_q5k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                       void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, xq, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q5_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, nullptr);
}

extern "C" int mmq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                       void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, xq, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q6_K, w, xq, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, nullptr);
}

extern "C" int mmq_q4k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                           void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, x, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q4_K, w, nullptr, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, x);
}

extern "C" int mmq_q5k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                           void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, x, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q5_K, w, nullptr, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, x);
}

extern "C" int mmq_q6k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                           void* ws, size_t ws_bytes, void* stream) {
  const int st = check_mmq(w, x, y, M, K, T, ws, ws_bytes);
  if (st != QMM_OK) return st;
  return mmq_dense(QMM_Q6_K, w, nullptr, y, M, K, T, ws, to_stream(stream), nullptr, nullptr, x);
}
