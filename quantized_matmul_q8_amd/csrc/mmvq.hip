// Decode matvec (MMVQ): y[t][i] = sum_k W[i][k] * x_t[k] for T <= 8 tokens,
// Q4_K, Q5_K or Q6_K weights against Q8_1 activations.
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
// Geometry for MI355X.  [8e] §2 describes the MMVQ geometry of a 48-SM
// LPDDR part (256 threads per row, one row per block) and its lesson: the
// kernel is latency-bound until enough loads are in flight.  Here:
// * one wave64 per weight row, eight rows per 512-thread workgroup (at
//   4096 rows every wave of the launch is resident at once, four per SIMD);
// * a wave reads its row as contiguous 16-byte pieces, so each load
//   instruction covers about 1 KB of consecutive row bytes (Q4_K / Q5_K:
//   plain 16-byte chunks of the row; Q6_K: 16 lanes per 210-byte block),
//   and re-deals the bytes to its lanes through LDS (per-wave rings or
//   regions, see each kernel); weight loads are non-temporal (each byte is
//   used once) and run a fixed number of rounds ahead of their use;
// * the activations of all T tokens are staged once per workgroup into LDS
//   as int8 payload plus, per 16 activations, the fp32 block scale and the
//   activation sum (the ones dots, computed once per workgroup instead of
//   once per row), so the eight rows share one read of them and per-unit
//   activation reads are LDS reads.  Each wave issues its staging loads
//   first and only one or two rounds of weight loads before the staging
//   barrier: staging loads queue behind every weight load the CU has already
//   issued, so a deep prefetch there would hold back the barrier and with it
//   all compute.  The weight and activation
//   pointers are deliberately not __restrict__: loads through restrict
//   pointers count as invariant and the compiler then moves them past the
//   barrier to their first use, serialising one HBM round trip per unit.
// When T*K is too large for the LDS budget the row is processed in K
// segments of equal length.  The row sum is a wave reduction; lane 0 writes
// y[t*M + row].
#include <algorithm>
#include <initializer_list>
#include <utility>

#include "qmm_common.hpp"

namespace qmm {

constexpr int kMmvqWaves = 8;             // rows per workgroup
constexpr int kMmvqThreads = 64 * kMmvqWaves;
constexpr int kMmvqLdsBudget = 68 * 1024; // bytes of staged activations per workgroup

// Issue priority from progress.  The SIMD arbiter prefers the oldest wave, so
// with equal work per wave the oldest waves (and the CU's first workgroup)
// run ahead and the youngest finish alone, with few loads in flight.  Each
// wave lowers its priority as it gets through its row (3 in the first
// quarter, 0 in the last), so waves that are behind are issued first and
// the waves of a CU finish together.  (Q4_K at T = 1 is balanced enough
// without and measures 2% faster so.)
template <bool ON = true>
__device__ __forceinline__ void progress_prio(int done, int total) {
  if constexpr (ON) {
    const int q = __builtin_amdgcn_readfirstlane((4 * done) / total);
    if (q <= 0) __builtin_amdgcn_s_setprio(3);
    else if (q == 1) __builtin_amdgcn_s_setprio(2);
    else if (q == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
}

// Per-slot routed-expert matvec (SLOT mode, T = 1): workgroup row block
// blockIdx.x of routed slot blockIdx.y = t * top_k + k multiplies expert
// ids[slot]'s rows (w + e * stride) with activation row t (rows_per_token
// == 1) or slot, into output row slot.  Each slot re-reads its expert's
// weights, which is what the grouped GEMM avoids.
struct SlotArgs {
  const int32_t* ids;
  int64_t stride;  // bytes between experts
  int E, top_k, rows_per_token;
};

// Expert weights, activation row and output row of this workgroup's slot;
// ids outside [0, E) are clamped (a documented precondition: no fault, but
// the row is meaningless).
__device__ __forceinline__ void slot_rebase(const SlotArgs& S, size_t xstride, int M, const uint8_t*& w,
                                            const uint8_t*& xq, float* __restrict__& y) {
  const int slot = blockIdx.y;
  const int e = min(max(S.ids[slot], 0), S.E - 1);
  w += static_cast<size_t>(e) * static_cast<size_t>(S.stride);
  xq += static_cast<size_t>(S.rows_per_token == 1 ? slot / S.top_k : slot) * xstride;
  y += static_cast<size_t>(slot) * M;
}

// Super-blocks per K segment: T tokens of staged activations must fit the
// LDS budget (1.5 bytes per activation) and the lane unit limit; the row is
// then split into segments of equal length (a short last segment would pay
// a whole staging round trip for a few blocks).
static int mmvq_chunk_blocks(int nb, int T, int units_per_block, int max_units) {
  int by_lds = kMmvqLdsBudget / (T * kQK * 3 / 2);
  int by_units = 64 * max_units / units_per_block;
  int c = by_lds < by_units ? by_lds : by_units;
  if (c < 1) c = 1;
  const int nseg = (nb + c - 1) / c;
  return (nb + nseg - 1) / nseg;
}

// Staged activations, in the order the lanes consume them (consecutive
// lanes read consecutive 16-byte slots, so the reads are free of bank
// conflicts).  Per token t and segment-local super-block bl, 384 bytes:
// * Q4_K, value chunk v = 0..7 (pair p = v/2, half h = v%2), index
//   i = (t*cb + bl)*8 + v in three arrays of 16-byte entries:
//     A[i]  activations 16h .. 16h+15 of Q8_1 block 2p   (low-nibble sub-block)
//     B[i]  the same of block 2p+1                        (high-nibble sub-block)
//     Z[i]  (d, S_h) of block 2p, (d, S_h) of block 2p+1 (fp32; S_h the sum of
//           the 16 activations, an integer dot against ones)
// * Q6_K, unit u = 0..3 (half h = u/2 of the super-block, 16-half l = u%2),
//   index i = (t*cb + bl)*4 + u in six arrays: P_g[i] (g = 0..3) the
//   activations 16l .. 16l+15 of Q8_1 block 4h + g, Z01[i] and Z23[i] the
//   (d, S_l) pairs of blocks 4h, 4h+1 and 4h+2, 4h+3.
// Each array holds T*cb*8 (Q4_K) or T*cb*4 (Q6_K) entries.
template <int FMT>
__device__ __forceinline__ uint4* stage_array(uint8_t* lds, int T, int cb, int a) {
  return reinterpret_cast<uint4*>(lds + static_cast<size_t>(a) * T * cb * (FMT == QMM_Q4_K ? 128 : 64));
}

// Load Q8_1 blocks [blk0, blk0 + nblk) of T tokens: this thread's r-th
// block.  The load is unconditional (out-of-range threads re-read block 0)
// so that no branch separates the staging loads from the weight loads that
// follow them.
__device__ __forceinline__ void stage_acts_load(const uint8_t* xq, size_t xstride, int T, int blk0,
                                                int nblk, int r, uint2 (&u)[5], int& t, int& j) {
  const int bi = threadIdx.x + kMmvqThreads * r;
  const int bc = bi < T * nblk ? bi : 0;
  t = bc / nblk;
  j = bc % nblk;
  const uint2* src = reinterpret_cast<const uint2*>(xq + t * xstride + static_cast<size_t>(blk0 + j) * kQ8Bytes);
#pragma unroll
  for (int k = 0; k < 5; ++k) u[k] = src[k];
}

// Store one loaded block into the staged layout.  Unconditional as well:
// threads past the end re-write block 0 of token 0 with the same bytes the
// owning thread writes.
template <int FMT>
__device__ __forceinline__ void stage_acts_store(uint8_t* lds, int T, int cb, const uint2 (&u)[5], int t, int j) {
  const uint4 half0 = make_uint4(u[0].y, u[1].x, u[1].y, u[2].x);
  const uint4 half1 = make_uint4(u[2].y, u[3].x, u[3].y, u[4].x);
  // activation sums of the two 16-halves as integer dots against ones ([8e] §2)
  int lo = dot4(0x01010101u, u[0].y, 0);
  lo = dot4(0x01010101u, u[1].x, lo);
  lo = dot4(0x01010101u, u[1].y, lo);
  lo = dot4(0x01010101u, u[2].x, lo);
  int hi = dot4(0x01010101u, u[2].y, 0);
  hi = dot4(0x01010101u, u[3].x, hi);
  hi = dot4(0x01010101u, u[3].y, hi);
  hi = dot4(0x01010101u, u[4].x, hi);
  const float d = h2f(u[0].x & 0xffffu);
  const int bl = j >> 3, s = j & 7;
  if constexpr (FMT == QMM_Q4_K) {
    const int p = s >> 1, par = s & 1;
    const size_t i0 = (static_cast<size_t>(t) * cb + bl) * 8 + 2 * p;  // value chunk v = 2p + h
    uint4* X = stage_array<FMT>(lds, T, cb, par);
    X[i0] = half0;
    X[i0 + 1] = half1;
    float2* Z = reinterpret_cast<float2*>(stage_array<FMT>(lds, T, cb, 2));
    Z[2 * i0 + par] = make_float2(d, static_cast<float>(lo));
    Z[2 * (i0 + 1) + par] = make_float2(d, static_cast<float>(hi));
  } else {
    const int h = s >> 2, g = s & 3;
    const size_t i0 = (static_cast<size_t>(t) * cb + bl) * 4 + 2 * h;  // unit u = 2h + l
    uint4* X = stage_array<FMT>(lds, T, cb, g);
    X[i0] = half0;
    X[i0 + 1] = half1;
    float2* Z = reinterpret_cast<float2*>(stage_array<FMT>(lds, T, cb, 4 + (g >> 1)));
    Z[2 * i0 + (g & 1)] = make_float2(d, static_cast<float>(lo));
    Z[2 * (i0 + 1) + (g & 1)] = make_float2(d, static_cast<float>(hi));
  }
}

// Q4_K and Q5_K rows are read as plain consecutive 16-byte chunks: lane l
// loads chunks l, l + 64, l + 128, ... of its row, so each wave load
// instruction covers 1 KB of contiguous bytes (the access pattern of the
// read-ceiling probe; loads of 16 bytes at a 32-byte stride or per-lane
// header loads cost 25-40% more time for the same bytes).  A 144-byte Q4_K
// block is exactly nine chunks: chunk 0 is the header (d, dmin, packed
// scales), chunk 1 + 2p + h holds value bytes 16 + 32p + 16h .. +15, i.e. 16
// weights of sub-block 2p (low nibbles) and 16 of sub-block 2p + 1 (high
// nibbles).  A 176-byte Q5_K block is eleven: the same header, then the two
// chunks of fifth bits qh[0..15] and qh[16..31], then the eight value
// chunks; value chunk (p, h) takes its fifth bits from qh chunk h (bits 2p
// and 2p + 1 of the bytes at the same positions).
//
// Rounds are consumed in load order.  In a round, header (and fifth-bit)
// chunks are copied to a per-wave ring of 16 block slots in LDS; then the
// (at most eight) headers that arrived in this round are decoded by all 64
// lanes at once, lane l taking sub-block l % 8 of the (l / 8)-th of them,
// into a ring of (d*sc, dmin*m) pairs; then each value chunk reads its two
// pairs with one 16-byte LDS read.  Every scale is thus decoded once per row
// instead of once per chunk, with no divergent decode path.  A block's
// header precedes its values and a value chunk's header lies in the same or
// the previous round (64 chunks > 11), so at most 15 blocks are live and 16
// slots never collide; one wave's LDS accesses execute in program order.
template <int FMT>
struct MvRow {
  static constexpr bool kQ5 = FMT == QMM_Q5_K;
  static constexpr int kBytes = kQ5 ? kQ5Bytes : kQ4Bytes;
  static constexpr int kChunks = kBytes / 16;               // 16-byte chunks per block: 9 or 11
  static constexpr int kVal0 = kQ5 ? 3 : 1;                 // first value chunk
  static constexpr int kRounds = kQ5 ? 8 : 7;               // 64-chunk rounds per segment (43 blocks fit)
  static constexpr int kSlot = 16 + (kQ5 ? 32 : 0) + 64;    // ring bytes per block: header, fifth bits, scales
};
constexpr int kQ4Ring = 16;   // block slots per wave in the header and scale rings
// Rounds in flight ahead of the one being consumed.  Issuing every round up
// front buys no memory parallelism (a CU's miss queue fills and the issue
// stalls) and delays the activation staging, which waits for all waves of
// the workgroup; two rounds ahead keep the queue full while computing.
constexpr int kQ4Ahead = 2;

// DEBUG == true: write the integer sub-block sums (D per (t, row, sub-block),
// S per (t, sub-block) from row 0) instead of the scaled result.  Same
// loads, unpacking and dot products; the two 16-weight halves of D are
// added with integer atomics into zeroed buffers.  Up to T = 6 the kernel
// is held to 128 VGPRs, four waves per SIMD (two workgroups per CU): Q5_K
// at T = 4 would otherwise take 130 VGPRs and T = 5, 6 take 139-172, each
// running one workgroup per CU (T = 4 15% and T = 5 20% slower so, even
// though the cap spills a few registers at T = 5, 6).
template <int FMT, int T, bool DEBUG, bool SLOT = false>
__global__ __launch_bounds__(kMmvqThreads) __attribute__((amdgpu_waves_per_eu(T <= 6 ? 4 : 1)))
void mmvq_q45k_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb, int cb,
                      int32_t* __restrict__ dbgD, int32_t* __restrict__ dbgS, SlotArgs SA) {
  using RL = MvRow<FMT>;
  constexpr int C = RL::kChunks;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_raw = blockIdx.x * kMmvqWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves load a valid row, store nothing
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  if constexpr (SLOT) slot_rebase(SA, xstride, M, w, xq, y);
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * RL::kBytes;
  const uint4* stA = stage_array<QMM_Q4_K>(lds, T, cb, 0);
  const uint4* stB = stage_array<QMM_Q4_K>(lds, T, cb, 1);
  const float4* stZ = reinterpret_cast<const float4*>(stage_array<QMM_Q4_K>(lds, T, cb, 2));
  uint8_t* rings = lds + static_cast<size_t>(T) * cb * 8 * 48 + static_cast<size_t>(wave) * kQ4Ring * RL::kSlot;
  uint4* hdr_ring = reinterpret_cast<uint4*>(rings);                  // [16] raw headers
  uint4* qh_ring = reinterpret_cast<uint4*>(rings + kQ4Ring * 16);    // Q5_K: [16][2] fifth-bit chunks
  float2* sc_ring = reinterpret_cast<float2*>(rings + kQ4Ring * (RL::kSlot - 64));  // [16][8] (d*sc, dmin*m)
  constexpr int RS = (T * 64 * 8 + kMmvqThreads - 1) / kMmvqThreads;  // staging rounds bound
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  for (int b0 = 0; b0 < nb; b0 += cb) {
    const int nbc = min(cb, nb - b0);
    const int nblk = nbc * 8;   // Q8_1 blocks in this segment
    const int nch = nbc * C;    // 16-byte chunks of the row in this segment
    // 1. activation staging loads (issued first)
    uint2 su[RS][5];
    int st[RS], sj[RS];
#pragma unroll
    for (int r = 0; r < RS; ++r) stage_acts_load(xq, xstride, T, b0 * 8, nblk, r, su[r], st[r], sj[r]);
    // 2. every chunk of this lane (unconditional loads; extra lanes re-read the last chunk)
    const uint8_t* seg = wrow + static_cast<size_t>(b0) * RL::kBytes;
    uint4 v[RL::kRounds];
#pragma unroll
    for (int r = 0; r < kQ4Ahead; ++r) v[r] = ld16_nt(seg + 16 * min(lane + 64 * r, nch - 1));
    __builtin_amdgcn_sched_barrier(0);
    // 3. publish the activations
    __syncthreads();  // previous segment's LDS reads are done
#pragma unroll
    for (int r = 0; r < RS; ++r) stage_acts_store<QMM_Q4_K>(lds, T, cb, su[r], st[r], sj[r]);
    if constexpr (DEBUG) {
      if (blockIdx.x == 0) {
#pragma unroll
        for (int r = 0; r < RS; ++r)
          dbgS[static_cast<size_t>(st[r]) * nb * 8 + b0 * 8 + sj[r]] = static_cast<int>(su[r][4].y);
      }
    }
    __syncthreads();
    // 4. consume the rounds in load order
    int bl = lane / C, k = lane - C * (lane / C);  // block and chunk-in-block of chunk lane + 64 r
#pragma unroll
    for (int r = 0; r < RL::kRounds; ++r) {
      if (r + kQ4Ahead < RL::kRounds) {
        v[r + kQ4Ahead] = ld16_nt(seg + 16 * min(lane + 64 * (r + kQ4Ahead), nch - 1));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (64 * r >= nch) break;                 // uniform: round entirely past the segment
      progress_prio<!(FMT == QMM_Q4_K && T == 1)>(b0 * C + 64 * r, nb * C);
      const bool ok = lane + 64 * r < nch;
      if (ok && k == 0) hdr_ring[bl % kQ4Ring] = v[r];  // header chunk
      if constexpr (RL::kQ5) {
        if (ok && (k == 1 || k == 2)) qh_ring[(bl % kQ4Ring) * 2 + (k - 1)] = v[r];  // fifth bits
      }
      {
        // headers of blocks ceil(64r / C) .. (64r + 63) / C arrived in this round
        const int bd = (64 * r + C - 1) / C + (lane >> 3), jd = lane & 7;
        if (bd <= (64 * r + 63) / C && bd < nbc) {
          const uint4 hdr = hdr_ring[bd % kQ4Ring];
          int sc, m;
          q4k_scale_min(jd, hdr.y, hdr.z, hdr.w, sc, m);
          sc_ring[(bd % kQ4Ring) * 8 + jd] =
              make_float2(h2f(hdr.x & 0xffffu) * static_cast<float>(sc), h2f(hdr.x >> 16) * static_cast<float>(m));
        }
      }
      if (ok && k >= RL::kVal0) {
        const int kv = k - RL::kVal0;  // value chunk 0..7
        const int p = kv >> 1, h = kv & 1;
        const float4 dsm = *reinterpret_cast<const float4*>(sc_ring + (bl % kQ4Ring) * 8 + 2 * p);
        const float ds0 = dsm.x, dm0 = dsm.y, ds1 = dsm.z, dm1 = dsm.w;
        const uint32_t qw[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        // 4-bit values of sub-blocks 2p (low nibbles) and 2p + 1 (high nibbles),
        // with the Q5_K fifth bits as bit 4 (0..31)
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          lo[i4] = qw[i4] & 0x0f0f0f0fu;
          hi[i4] = (qw[i4] >> 4) & 0x0f0f0f0fu;
        }
        if constexpr (RL::kQ5) {
          const uint4 qhv = qh_ring[(bl % kQ4Ring) * 2 + h];
          const uint32_t qh[4] = {qhv.x, qhv.y, qhv.z, qhv.w};
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            lo[i4] |= ((qh[i4] >> (2 * p)) & 0x01010101u) << 4;
            hi[i4] |= ((qh[i4] >> (2 * p + 1)) & 0x01010101u) << 4;
          }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const size_t i = (static_cast<size_t>(t) * cb + bl) * 8 + kv;
          const uint4 xa = stA[i];  // 16 activations of sub-block 2p
          const uint4 xc = stB[i];  // 16 activations of sub-block 2p+1
          const float4 z = stZ[i];  // (d, S_h) of 2p, (d, S_h) of 2p+1
          const uint32_t x0[4] = {xa.x, xa.y, xa.z, xa.w};
          const uint32_t x1[4] = {xc.x, xc.y, xc.z, xc.w};
          int D0 = 0, D1 = 0;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            D0 = dot4(lo[i4], x0[i4], D0);  // sub-block 2p
            D1 = dot4(hi[i4], x1[i4], D1);  // sub-block 2p+1
          }
          if constexpr (DEBUG) {
            if (row_ok) {
              const int sb0 = b0 * 8 + bl * 8 + 2 * p;
              int32_t* Dt = dbgD + (static_cast<size_t>(t) * M + row) * (nb * 8);
              atomicAdd(Dt + sb0, D0);
              atomicAdd(Dt + sb0 + 1, D1);
            }
          } else {
            acc[t] += z.x * (ds0 * static_cast<float>(D0) - dm0 * z.y) +
                      z.z * (ds1 * static_cast<float>(D1) - dm1 * z.w);
          }
        }
      }
      // chunk lane + 64 (r + 1)
      bl += 64 / C;
      k += 64 % C;
      if (k >= C) { k -= C; ++bl; }
      // opaque, so the unrolled rounds do not precompute (and keep live)
      // every round's ring and staging addresses from the start; Q4_K at
      // T = 1 fits four waves per SIMD either way and runs faster without,
      // except in slot mode (short rows: 1.45x slower without)
      if constexpr (T >= 2 || RL::kQ5 || SLOT) __asm__ volatile("" : "+v"(bl), "+v"(k));
    }
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && row_ok) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

// Q6_K rows are read as consecutive 16-byte pieces: 16 lanes per 210-byte
// block, lane j of a block loading bytes 16j .. 16j+15 for j < 13 and bytes
// 194 .. 209 for j = 13 (lanes 14, 15 idle), so one wave load instruction
// covers four consecutive blocks (840 contiguous bytes) instead of scattered
// pieces of sixteen (blocks are 2-byte aligned; gfx950 serves unaligned
// 16-byte loads).  Rounds of loads are issued in order, a fixed number
// ahead of the chunk being multiplied, and only kQ6Pre of them before the
// activation staging: staging loads queue behind every weight load the CU
// has already issued, so a deep prefetch there delays the staging barrier
// (and with it all compute) until most of the matrix has arrived.
// The pieces of 16 blocks at a time are written to a wave-private LDS region
// (one 16-byte slot per piece, blocks kQ6BlkStride bytes apart so that the
// reads below are free of bank conflicts), from where lane l takes its unit:
// block l/4, half h = (l%4)/2 and 16-half hf = l%2 of it, i.e. 64 weights in
// four 16-weight sub-blocks (g = 0..3 at positions 128h + 32g + 16hf + i).
// Bytes used: ql[64h + 16hf ..+16] (g = 0, 2), ql[64h + 32 + 16hf ..+16]
// (g = 1, 3), qh[32h + 16hf ..+16], sc[8h .. 8h+7] and d.
constexpr int kQ6Chunk = 16;       // blocks per LDS chunk: 64 units, one per lane
constexpr int kQ6BlkStride = 272;  // LDS bytes per block in the piece region
// piece rounds per segment held in registers: 16 (64 blocks) for T <= 2,
// fewer where the staged activations of more tokens shorten the segment
__host__ __device__ constexpr int q6_rounds(int T) { return T <= 2 ? 16 : (T <= 4 ? 8 : 4); }
constexpr int kQ6WaveRegion = kQ6Chunk * kQ6BlkStride;
constexpr int kQ6Pre = 1;    // piece rounds issued before the activation staging
constexpr int kQ6Ahead = 4;  // piece rounds issued ahead of the chunk being multiplied

__device__ __forceinline__ uint4 ld16_u(const uint8_t* p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);  // one dwordx4 load at a 2-byte aligned address
  return v;
}

template <int T, bool DEBUG, bool SLOT = false>
__global__ __launch_bounds__(kMmvqThreads) void mmvq_q6k_kernel(const uint8_t* w, const uint8_t* xq,
                                                                float* __restrict__ y, int M, int nb,
                                                                int cb, int32_t* __restrict__ dbgD, SlotArgs SA) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_raw = blockIdx.x * kMmvqWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  if constexpr (SLOT) slot_rebase(SA, xstride, M, w, xq, y);
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * kQ6Bytes;
  uint8_t* wreg = lds + static_cast<size_t>(T) * cb * 8 * 48 + wave * kQ6WaveRegion;
  constexpr int RS = (T * 64 * 8 + kMmvqThreads - 1) / kMmvqThreads;
  const int pj = lane & 15, pb = lane >> 4;         // piece of a block, block within a round
  const int poff = pj < 13 ? 16 * pj : 194;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;

  for (int b0 = 0; b0 < nb; b0 += cb) {
    const int nbc = min(cb, nb - b0);
    const int nblk = nbc * 8;
    // 1. activation staging loads, then every weight piece of the segment
    uint2 su[RS][5];
    int st[RS], sj[RS];
#pragma unroll
    for (int r = 0; r < RS; ++r) stage_acts_load(xq, xstride, T, b0 * 8, nblk, r, su[r], st[r], sj[r]);
    constexpr int NR = q6_rounds(T);
    uint4 pc[NR];
    // pieces of round r (blocks 4r .. 4r+3); a round past the segment is skipped
    auto load_round = [&](int r) {
      pc[r] = make_uint4(0u, 0u, 0u, 0u);
      if (4 * r < nbc && pj < 14 && 4 * r + pb < nbc)
        pc[r] = ld16_u(wrow + static_cast<size_t>(b0 + 4 * r + pb) * kQ6Bytes + poff);
    };
#pragma unroll
    for (int r = 0; r < kQ6Pre && r < NR; ++r) load_round(r);
    __builtin_amdgcn_sched_barrier(0);
    // 2. publish the activations
    __syncthreads();  // previous segment's LDS reads are done
#pragma unroll
    for (int r = 0; r < RS; ++r) stage_acts_store<QMM_Q6_K>(lds, T, cb, su[r], st[r], sj[r]);
    __syncthreads();
    // 3. chunks of 16 blocks: pieces to the wave's region, then one unit per lane
#pragma unroll
    for (int ch = 0; ch < NR / 4; ++ch) {
      if (16 * ch >= nbc) break;  // uniform
      progress_prio(b0 + 16 * ch, nb);
      {
        // rounds up to kQ6Ahead past this chunk, not issued yet
        const int lo = ch == 0 ? kQ6Pre : 4 * ch + kQ6Ahead;
        const int lo2 = lo > kQ6Pre ? lo : kQ6Pre;
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (r >= lo2 && r < 4 * ch + 4 + kQ6Ahead) load_round(r);
        __builtin_amdgcn_sched_barrier(0);
      }
      // (this wave's reads of the previous chunk precede these writes in program order)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (pj < 14) *reinterpret_cast<uint4*>(wreg + (4 * q + pb) * kQ6BlkStride + 16 * pj) = pc[4 * ch + q];
      const int bl = 16 * ch + (lane >> 2);  // segment-local block of this lane's unit
      if (bl < nbc) {
        const uint8_t* blk = wreg + (lane >> 2) * kQ6BlkStride;
        const int c = lane & 3, h = c >> 1, half16 = c & 1;
        const uint4 qa = *reinterpret_cast<const uint4*>(blk + 16 * (4 * h + half16));      // g = 0, 2
        const uint4 qb = *reinterpret_cast<const uint4*>(blk + 16 * (4 * h + 2 + half16));  // g = 1, 3
        const uint4 qh = *reinterpret_cast<const uint4*>(blk + 16 * (8 + 2 * h + half16));  // bit pairs
        const uint2 scs = *reinterpret_cast<const uint2*>(blk + 192 + 8 * h);               // sc[8h .. 8h+7]
        const float d = h2f(*reinterpret_cast<const uint16_t*>(blk + 16 * 13 + 14));        // byte 208
        float dsc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // sc[8h + 2g + half16]: byte (2g + half16) of the 8 loaded bytes
          const uint32_t word = g < 2 ? scs.x : scs.y;
          const int sc = static_cast<int8_t>((word >> (8 * (2 * (g & 1) + half16))) & 0xffu);
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
          const size_t ix = (static_cast<size_t>(t) * cb + bl) * 4 + c;
          const float4 z01 = reinterpret_cast<const float4*>(stage_array<QMM_Q6_K>(lds, T, cb, 4))[ix];
          const float4 z23 = reinterpret_cast<const float4*>(stage_array<QMM_Q6_K>(lds, T, cb, 5))[ix];
          const float zd[4] = {z01.x, z01.z, z23.x, z23.z}, zs[4] = {z01.y, z01.w, z23.y, z23.w};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint4 xv = stage_array<QMM_Q6_K>(lds, T, cb, g)[ix];  // activations of block 4h+g, half
            int D = dot4(q6[g][0], xv.x, 0);
            D = dot4(q6[g][1], xv.y, D);
            D = dot4(q6[g][2], xv.z, D);
            D = dot4(q6[g][3], xv.w, D);
            // sum (q6 - 32) * q = D - 32 * S_half, exact in fp32 (|.| < 2^24)
            const float D6 = static_cast<float>(D) - 32.0f * zs[g];
            if constexpr (DEBUG) {
              if (row_ok)
                dbgD[(static_cast<size_t>(t) * M + row) * (nb * 16) + (b0 * 8 + bl * 8 + 4 * h + g) * 2 + half16] =
                    static_cast<int>(D6);
            } else {
              acc[t] += zd[g] * dsc[g] * D6;
            }
          }
        }
      }
    }
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && row_ok) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

// One token (T = 1), Q4_K and Q5_K.  The whole matrix is one read, so the
// time is set by how early and how many weight bytes are in flight.  Each
// wave copies its row segment straight into its own LDS region with
// global_load_lds (kRounds copies of 1 KB, all issued at the start: a deep
// prefetch that holds no registers), after the workgroup's copy of the raw
// Q8_1 activation blocks of the segment.  Lane l then takes unit 64u + l of
// the segment -- super-block b = unit / 4, sub-block pair p = unit % 4: the
// 32 value bytes 16 + 32p .. 16 + 32p + 31 (Q5_K: 48 + 32p, plus the 32
// fifth-bit bytes), i.e. all 32 weights of sub-blocks 2p (low nibbles) and
// 2p + 1 (high nibbles) -- decodes their two scales and mins from the
// header itself and multiplies them with Q8_1 blocks 8b + 2p and 8b + 2p + 1,
// whose stored integer sums give the min term ([8e] §2).  Unit round u
// waits only for the copies that hold its 16 super-blocks, so it runs while
// later rounds are still arriving; no lane takes a divergent path.

template <int FMT>
struct MvDma {
  static constexpr bool kQ5 = FMT == QMM_Q5_K;
  static constexpr int kBytes = kQ5 ? kQ5Bytes : kQ4Bytes;
  static constexpr int kRounds = kQ5 ? 8 : 7;       // 1 KB copies per wave per segment
  static constexpr int kMaxBlocks = kQ5 ? 46 : 48;  // super-blocks per segment (3 unit rounds)
  static constexpr int kUnitRounds = 3;
  static_assert(kMaxBlocks * kBytes <= kRounds * 1024 && 4 * kMaxBlocks <= 64 * kUnitRounds, "segment");
  static constexpr int kQ8Seg = 8 * kQ8Bytes;       // Q8_1 bytes per super-block (320)
  // copies still allowed in flight when unit round u starts: those past the
  // last byte of its super-blocks (every copy is issued at the start: a
  // schedule that issues later copies after the first unit rounds, or a
  // barrier between copy rounds so they are issued round by round across the
  // waves, measured no faster; the memory system serves the requests of all
  // CUs in about the order they arrive)
  static constexpr int in_flight(int u) {
    const int b = 16 * (u + 1) < kMaxBlocks ? 16 * (u + 1) : kMaxBlocks;
    const int need = (b * kBytes + 1023) / 1024;
    return kRounds - (need < kRounds ? need : kRounds);
  }
};

// Unit (super-block at blk in LDS, sub-block pair p) of a Q4_K / Q5_K row:
// the 4-bit values (Q5_K: with the fifth bit as bit 4) of sub-blocks 2p (lo)
// and 2p + 1 (hi), four per dword, and their integer scales and mins.
struct Q45Unit {
  uint32_t lo[8], hi[8];
  uint32_t scm;  // bytes: scale of sub-block 2p, of 2p + 1, min of 2p, of 2p + 1 (6 bits each)
  uint32_t dd;   // f16 d | f16 dmin << 16
};

// Scales and mins of sub-blocks 2p and 2p + 1 from the 12 packed bytes
// S = (s0, s1, s2) of a Q4_K / Q5_K header, as the bytes of one dword (the
// packing of q4k_scale_min, for both sub-blocks at once, with byte
// permutes whose selectors depend only on p):
//   p < 2 (j = 2p, 2p + 1 < 4):  sc = S[j] & 63,  m = S[j + 4] & 63
//   p >= 2 (j >= 4):  sc = S[j + 4] & 15 | (S[j - 4] >> 6) << 4,
//                     m  = S[j + 4] >> 4 | (S[j] >> 6) << 4
__device__ __forceinline__ uint32_t q4k_scale_min_pair(int p, uint32_t s0, uint32_t s1, uint32_t s2) {
  const uint32_t b = 2u * (p & 1);                       // first byte of the pair within its dword
  const uint32_t selx = b | (b + 1) << 8 | (b + 4) << 16 | (b + 5) << 24;
  const uint32_t sely = p < 2 ? 0x0c0c0c0cu : (b | (b + 1) << 8 | b << 16 | (b + 1) << 24);  // 0x0c: zero
  const uint32_t x = __builtin_amdgcn_perm(s1, s0, selx);  // S[j - 4 or j], S[j or j + 4] (p >= 2 / p < 2)
  const uint32_t yv = __builtin_amdgcn_perm(s2, s2, sely); // S[j + 4] twice (p >= 2), else 0
  const uint32_t hi = p < 2 ? (x & 0x3f3f3f3fu) : ((x >> 2) & 0x30303030u);
  return hi | (yv & 0x00000f0fu) | ((yv >> 4) & 0x0f0f0000u);
}
template <int FMT>
__device__ __forceinline__ void q45_unit(const uint8_t* blk, int p, Q45Unit& U) {
  constexpr bool kQ5 = FMT == QMM_Q5_K;
  const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
  U.scm = q4k_scale_min_pair(p, hdr.y, hdr.z, hdr.w);
  U.dd = hdr.x;
  const uint8_t* qv = blk + (kQ5 ? 48 : 16) + 32 * p;
  const uint4 qa = *reinterpret_cast<const uint4*>(qv);
  const uint4 qb = *reinterpret_cast<const uint4*>(qv + 16);
  const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    U.lo[k] = qw[k] & 0x0f0f0f0fu;
    U.hi[k] = (qw[k] >> 4) & 0x0f0f0f0fu;
  }
  if constexpr (kQ5) {
    // fifth bit of weight i of sub-block j: bit j of byte i of bytes 16 .. 47
    const uint4 ha = *reinterpret_cast<const uint4*>(blk + 16);
    const uint4 hb = *reinterpret_cast<const uint4*>(blk + 32);
    const uint32_t hw[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      U.lo[k] |= ((hw[k] >> (2 * p)) & 0x01010101u) << 4;
      U.hi[k] |= ((hw[k] >> (2 * p + 1)) & 0x01010101u) << 4;
    }
  }
}

// The unit against one token's Q8_1 blocks 8b + 2p, 8b + 2p + 1 (raw 40-byte
// blocks): the integer sums D, each started at the bits
// of 1.5 * 2^23 (X = that bit pattern + D; |D| <= 32 * 31 * 128 < 2^22), and
// the blocks' stored sums S and scales.
struct Q45Dot {
  int X0, X1, S0, S1;
  float dx0, dx1;
  __device__ __forceinline__ int D0() const { return X0 - static_cast<int>(kMagicBits); }
  __device__ __forceinline__ int D1() const { return X1 - static_cast<int>(kMagicBits); }
};
// The two blocks (80 bytes at xu, 16-byte aligned) are read as five 16-byte
// chunks: block 2p has d at byte 0, values at 4 .. 35 and its sum at 36,
// block 2p + 1 the same 40 bytes on.  Consecutive units are 80 bytes apart,
// so eight lanes' chunks cover all 32 banks (8-byte reads hit each bank
// twice).
__device__ __forceinline__ Q45Dot q45_dot_c(const Q45Unit& U, const uint8_t* xu) {
  const uint4* c = reinterpret_cast<const uint4*>(xu);
  const uint4 c0 = c[0], c1 = c[1], c2 = c[2], c3 = c[3], c4 = c[4];
  const uint32_t xa[8] = {c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w, c2.x};
  const uint32_t xc[8] = {c2.w, c3.x, c3.y, c3.z, c3.w, c4.x, c4.y, c4.z};
  Q45Dot r;
  r.X0 = dot4_magic(U.lo[0], xa[0]);
  r.X1 = dot4_magic(U.hi[0], xc[0]);
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    r.X0 = dot4(U.lo[k], xa[k], r.X0);
    r.X1 = dot4(U.hi[k], xc[k], r.X1);
  }
  r.S0 = static_cast<int>(c2.y);
  r.S1 = static_cast<int>(c4.w);
  r.dx0 = h2f(c0.x & 0xffffu);
  r.dx1 = h2f(c2.z & 0xffffu);
  return r;
}

// Per-unit factors of the float combine, shared by every token: a = d*sc,
// c = -a * 1.5 * 2^23 (exact: a has at most 17 significant bits), b =
// -dmin*m, for sub-blocks 2p and 2p + 1.
struct Q45Coef {
  float a0, a1, c0, c1, b0, b1;
};
__device__ __forceinline__ Q45Coef q45_coef(const Q45Unit& U) {
  const float d = h2f(U.dd & 0xffffu), dmin = h2f(U.dd >> 16);
  Q45Coef C;
  C.a0 = d * static_cast<float>(U.scm & 0xffu);
  C.a1 = d * static_cast<float>((U.scm >> 8) & 0xffu);
  C.c0 = -C.a0 * kMagic;
  C.c1 = -C.a1 * kMagic;
  C.b0 = -(dmin * static_cast<float>((U.scm >> 16) & 0xffu));
  C.b1 = -(dmin * static_cast<float>(U.scm >> 24));
  return C;
}

// acc + the unit's y contribution for one token, dx * (d*sc*D - dmin*m*S) for
// both sub-blocks: d*sc*D in one fma from the biased sum, then the min term
// and the activation scale in one fma each.
__device__ __forceinline__ float q45_accum(const Q45Coef& C, const Q45Dot& r, float acc) {
  const float t0 = __builtin_fmaf(C.b0, static_cast<float>(r.S0), __builtin_fmaf(C.a0, __int_as_float(r.X0), C.c0));
  const float t1 = __builtin_fmaf(C.b1, static_cast<float>(r.S1), __builtin_fmaf(C.a1, __int_as_float(r.X1), C.c1));
  return __builtin_fmaf(r.dx1, t1, __builtin_fmaf(r.dx0, t0, acc));
}

// Workgroup blk of the one-token Q4_K / Q5_K matvec (rows 8 blk .. 8 blk + 7),
// with the workgroup's LDS at lds.
template <int FMT, bool DEBUG>
__device__ __forceinline__ void q45_t1_body(uint8_t* lds, int blk, const uint8_t* w, const uint8_t* xq,
                                            float* __restrict__ y, int M, int nb, int cb,
                                            int32_t* __restrict__ dbgD, int32_t* __restrict__ dbgS) {
  using DL = MvDma<FMT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_raw = blk * kMmvqWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves read a valid row, store nothing
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * DL::kBytes;
  const uint8_t* wl = lds + wave * DL::kRounds * 1024;  // this wave's copy of its row segment
  const uint8_t* xl = lds + kMmvqWaves * DL::kRounds * 1024;  // the segment's raw Q8_1 blocks
  const uint32_t wl_a = lds_addr(wl), xl_a = lds_addr(xl);
  float acc = 0.0f;
  for (int b0 = 0; b0 < nb; b0 += cb) {
    const int nbc = min(cb, nb - b0);
    if (b0 > 0) __syncthreads();  // every wave is done with the previous segment's copies
    // 1. the activation blocks of the segment (nbc * 320 contiguous bytes), copies i = wave + 8k
    const int xs = nbc * (DL::kQ8Seg / 16);
    const uint8_t* xseg = xq + static_cast<size_t>(b0) * DL::kQ8Seg;
    for (int i = wave; 64 * i < xs; i += kMmvqWaves) dma16(xseg + 16 * min(64 * i + lane, xs - 1), xl_a + 1024 * i);
    // 2. the row segment, 16 bytes per lane per copy (lanes past its end
    // re-read its last 16 bytes)
    const int nch = nbc * (DL::kBytes / 16);
    const uint8_t* wseg = wrow + static_cast<size_t>(b0) * DL::kBytes;
#pragma unroll
    for (int r = 0; r < DL::kRounds; ++r) dma16<true>(wseg + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
    // 3. this wave's activation copies (issued first) are done; then everyone's
    wait_vmcnt<DL::kRounds>();
    __syncthreads();
    // 4. unit rounds
#pragma unroll
    for (int u = 0; u < DL::kUnitRounds; ++u) {
      if (u == 0) wait_vmcnt<DL::in_flight(0)>();  // (u is a constant once unrolled)
      else if (u == 1) wait_vmcnt<DL::in_flight(1)>();
      else wait_vmcnt<DL::in_flight(2)>();
      const int n = 64 * u + lane, b = n >> 2, p = n & 3;
      if (b < nbc) {  // (a unit round past the segment has no lanes: its waits stay in step)
        Q45Unit U;
        q45_unit<FMT>(wl + b * DL::kBytes, p, U);
        // Q8_1 blocks 8b + 2p and 8b + 2p + 1: f16 d, pad, q[32], int32 sum
        const Q45Dot r = q45_dot_c(U, xl + (8 * b + 2 * p) * kQ8Bytes);
        if constexpr (DEBUG) {
          const int sb = (b0 + b) * 8 + 2 * p;
          if (row_ok) {
            int32_t* Dr = dbgD + static_cast<size_t>(row) * (nb * 8);
            Dr[sb] = r.D0();
            Dr[sb + 1] = r.D1();
          }
          if (row_raw == 0) {
            dbgS[sb] = r.S0;
            dbgS[sb + 1] = r.S1;
          }
        } else {
          acc = q45_accum(q45_coef(U), r, acc);
        }
      }
    }
    // no copy may still be writing LDS when the next segment reuses it or
    // the workgroup ends
    wait_vmcnt<0>();
  }
  if constexpr (!DEBUG) {
    const float s = wave_sum(acc);
    if (lane == 0 && row_ok) y[row] = s;
  }
}

template <int FMT, bool DEBUG>
__global__ __launch_bounds__(kMmvqThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_q45k_t1_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb, int cb,
                         int32_t* __restrict__ dbgD, int32_t* __restrict__ dbgS) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  q45_t1_body<FMT, DEBUG>(lds, blockIdx.x, w, xq, y, M, nb, cb, dbgD, dbgS);
}

// LDS of the one-token Q4_K / Q5_K matvec: the eight row regions and the
// activation segment of cb super-blocks.
template <int FMT>
static size_t t1_lds_bytes(int cb) {
  using DL = MvDma<FMT>;
  return static_cast<size_t>(kMmvqWaves) * DL::kRounds * 1024 +
         (static_cast<size_t>(cb) * DL::kQ8Seg + 1023) / 1024 * 1024;
}

// Super-blocks per segment of the one-token Q4_K / Q5_K matvec (equal
// segments of at most kMaxBlocks).
template <int FMT>
static int t1_seg_blocks(int nb) {
  using DL = MvDma<FMT>;
  const int nseg = (nb + DL::kMaxBlocks - 1) / DL::kMaxBlocks;
  return (nb + nseg - 1) / nseg;
}

template <int FMT, bool DEBUG>
static int launch_mmvq_t1(const void* w, const void* xq, float* y, int M, int nb, int32_t* D, int32_t* S,
                          hipStream_t st) {
  using DL = MvDma<FMT>;
  const int cb = t1_seg_blocks<FMT>(nb);
  const size_t lds = t1_lds_bytes<FMT>(cb);
  static bool attr_set = false;
  if (!attr_set) {
    const size_t lmax = t1_lds_bytes<FMT>(DL::kMaxBlocks);
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_q45k_t1_kernel<FMT, DEBUG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lmax)) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((M + kMmvqWaves - 1) / kMmvqWaves), block(kMmvqThreads);
  hipLaunchKernelGGL((mmvq_q45k_t1_kernel<FMT, DEBUG>), grid, block, lds, st, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), y, M, nb, cb, D, S);
  return launch_status();
}

// Two to four tokens, Q4_K and Q5_K: the one-token design with one 16-wave workgroup
// per CU, so the T tokens' raw activation blocks (13.8 KB per token at
// K = 11008) are copied once per CU.  To fit them beside sixteen row
// segments, a wave's copies write only the row's own bytes: the copies past
// the segment are issued with their lanes masked off (a copy with no byte
// left keeps lane 0 on a 16-byte dummy slot, so every wave issues the same
// number of copies and the vmcnt waits stay exact).  Each lane decodes its
// unit once and multiplies it with every token.
// Q5_K works the same way with its 176-byte blocks (a segment of at most 46
// super-blocks in 8 copies).
constexpr int kTnWaves = 16;
constexpr int kTnEarly = 4;       // copies issued before the activation barrier (Q4_K: measured 3 .. 5 of 7)
constexpr int kLdsMax = 160 * 1024;

template <int FMT>
static int tn_max_blocks(int T) {
  using DL = MvDma<FMT>;
  const int by_lds = (kLdsMax - kTnWaves * 16) / (kTnWaves * DL::kBytes + T * 8 * kQ8Bytes);
  return by_lds < DL::kMaxBlocks ? by_lds : DL::kMaxBlocks;
}

template <int FMT, int T, bool DEBUG>
__global__ __launch_bounds__(64 * kTnWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_q45k_tn_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb, int cb,
                         int32_t* __restrict__ dbgD, int32_t* __restrict__ dbgS) {
  using DL = MvDma<FMT>;
  constexpr int kTnRounds = DL::kRounds;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_raw = blockIdx.x * kTnWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves read a valid row, store nothing
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  const uint8_t* wrow = w + static_cast<size_t>(row) * nb * DL::kBytes;
  const int wreg = cb * DL::kBytes;                                     // bytes per wave region
  const uint8_t* wl = lds + wave * wreg;
  const uint8_t* xl = lds + kTnWaves * wreg;                           // T tokens' raw Q8_1 blocks
  const uint32_t wl_a = lds_addr(wl), xl_a = lds_addr(xl);
  const uint32_t dummy_a = lds_addr(lds + kTnWaves * wreg + T * cb * 8 * kQ8Bytes) + 16 * wave;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  for (int b0 = 0; b0 < nb; b0 += cb) {
    const int nbc = min(cb, nb - b0);
    if (b0 > 0) __syncthreads();  // every wave is done with the previous segment's copies
    // 1. the activation blocks of the segment, token after token (nbc * 320 bytes each)
    const int tseg = nbc * (DL::kQ8Seg / 16), xs = T * tseg;  // 16-byte slots
    for (int i = wave; 64 * i < xs; i += kTnWaves) {
      const int sl = 64 * i + lane;
      if (sl < xs) {
        const int t = sl / tseg, j = sl - t * tseg;
        dma16(xq + t * xstride + static_cast<size_t>(b0) * DL::kQ8Seg + 16 * j, xl_a + 1024 * i);
      }
    }
    // 2. the row segment: lanes past its end are masked off
    const int nch = nbc * (DL::kBytes / 16);
    const uint8_t* wseg = wrow + static_cast<size_t>(b0) * DL::kBytes;
    auto copy_round = [&](int r) {
      const bool full = 64 * r < nch;
      if (full ? 64 * r + lane < nch : lane == 0)
        dma16<true>(wseg + 16 * min(64 * r + lane, nch - 1), full ? wl_a + 1024 * r : dummy_a);
    };
#pragma unroll
    for (int r = 0; r < kTnEarly; ++r) copy_round(r);
    // 3. this wave's activation copies (issued first) are done; then everyone's;
    //    then the rest of the row segment
    wait_vmcnt<kTnEarly>();
    __syncthreads();
#pragma unroll
    for (int r = kTnEarly; r < kTnRounds; ++r) copy_round(r);
    // 4. unit rounds
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      if (u == 0) wait_vmcnt<DL::in_flight(0)>();  // (u is a constant once unrolled)
      else if (u == 1) wait_vmcnt<DL::in_flight(1)>();
      else wait_vmcnt<DL::in_flight(2)>();
      const int n = 64 * u + lane, b = n >> 2, p = n & 3;
      if (b < nbc) {
        Q45Unit U;
        q45_unit<FMT>(wl + b * DL::kBytes, p, U);
        const Q45Coef C = q45_coef(U);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const Q45Dot r = q45_dot_c(U, xl + t * (nbc * DL::kQ8Seg) + (8 * b + 2 * p) * kQ8Bytes);
          if constexpr (DEBUG) {
            const int sb = (b0 + b) * 8 + 2 * p;
            if (row_ok) {
              int32_t* Dr = dbgD + (static_cast<size_t>(t) * M + row) * (nb * 8);
              Dr[sb] = r.D0();
              Dr[sb + 1] = r.D1();
            }
            if (row_raw == 0) {
              dbgS[static_cast<size_t>(t) * nb * 8 + sb] = r.S0;
              dbgS[static_cast<size_t>(t) * nb * 8 + sb + 1] = r.S1;
            }
          } else {
            acc[t] = q45_accum(C, r, acc[t]);
          }
        }
      }
    }
    wait_vmcnt<0>();  // nothing may still write LDS when it is reused or the workgroup ends
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && row_ok) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

template <int FMT, int T, bool DEBUG>
static int launch_mmvq_q45k_tn(const void* w, const void* xq, float* y, int M, int nb, int32_t* D, int32_t* S,
                               hipStream_t st) {
  using DL = MvDma<FMT>;
  const int cmax = tn_max_blocks<FMT>(T);
  const int nseg = (nb + cmax - 1) / cmax;
  const int cb = (nb + nseg - 1) / nseg;
  const size_t lds = static_cast<size_t>(kTnWaves) * cb * DL::kBytes + static_cast<size_t>(T) * cb * 8 * kQ8Bytes +
                     kTnWaves * 16;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_q45k_tn_kernel<FMT, T, DEBUG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((M + kTnWaves - 1) / kTnWaves), block(64 * kTnWaves);
  hipLaunchKernelGGL((mmvq_q45k_tn_kernel<FMT, T, DEBUG>), grid, block, lds, st, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), y, M, nb, cb, D, S);
  return launch_status();
}

static size_t mmvq_lds_bytes(int T, int cb) { return static_cast<size_t>(T) * cb * 8 * 48; }

template <bool DEBUG, int FMT = QMM_Q4_K>
static int launch_mmvq_q4k(const void* w, const void* xq, float* y, int M, int nb, int T,
                           int32_t* D, int32_t* S, hipStream_t st, const SlotArgs* slots = nullptr,
                           int nslots = 0) {
  using RL = MvRow<FMT>;
  // segment: whole blocks whose chunks fit the lane rounds, within the LDS budget
  const int cb = mmvq_chunk_blocks(nb, T, RL::kChunks, RL::kRounds);
  const dim3 grid((M + kMmvqWaves - 1) / kMmvqWaves), block(kMmvqThreads);
  const SlotArgs SA = slots ? *slots : SlotArgs{};
  const size_t lds = mmvq_lds_bytes(T, cb) + static_cast<size_t>(kMmvqWaves) * kQ4Ring * RL::kSlot;
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint8_t* xp = static_cast<const uint8_t*>(xq);
  if (!slots && T == 1) return launch_mmvq_t1<FMT, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 2) return launch_mmvq_q45k_tn<FMT, 2, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 3) return launch_mmvq_q45k_tn<FMT, 3, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 4) return launch_mmvq_q45k_tn<FMT, 4, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 5) return launch_mmvq_q45k_tn<FMT, 5, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 6) return launch_mmvq_q45k_tn<FMT, 6, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 7) return launch_mmvq_q45k_tn<FMT, 7, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (!slots && T == 8) return launch_mmvq_q45k_tn<FMT, 8, DEBUG>(w, xq, y, M, nb, D, S, st);
  if (slots) {
    if (DEBUG || T != 1) return QMM_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((mmvq_q45k_kernel<FMT, 1, false, true>), dim3(grid.x, nslots), block, lds, st, wp, xp, y,
                       M, nb, cb, D, S, SA);
    return launch_status();
  }
  switch (T) {
#define QMM_CASE(TT) \
  case TT: hipLaunchKernelGGL((mmvq_q45k_kernel<FMT, TT, DEBUG>), grid, block, lds, st, wp, xp, y, M, nb, cb, D, S, SA); break;
    QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
    default: return QMM_ERR_SHAPE;
  }
  return launch_status();
}

// One token, Q6_K: the one-token Q4_K design adapted to 210-byte blocks.
// A wave's row starts at any even byte, so it is copied as the 16-byte
// aligned chunks that cover it (the row's offset in its first chunk is
// `shift`); the first 8 KB (all of super-blocks 0 .. 37 for any shift) go
// straight into the wave's LDS region with global_load_lds, and the rest of
// the row (at most 8 more super-blocks) is loaded into registers, two 16-byte
// chunks per lane, issued after the copies and written over the region's
// first 2 KB (super-blocks 0 .. 9, done with by then) just before the last
// unit round.  Lane l takes unit 64u + l: super-block b = unit / 4, half
// h = (unit / 2) % 2 and 16-half q = unit % 2 of it, i.e. weights
// 128h + 32k + l for l in [16q, 16q + 16) and k = 0 .. 3 -- the bytes
// ql[64h + 16q ..], ql[64h + 32 + 16q ..] and qh[32h + 16q ..] (16 each), the
// scales sc[8h + 2k + q] and d -- against half q of Q8_1 blocks 8b + 4h + k.
// The signed values q6 - 32 are formed with a byte table lookup on the two
// high bits, so no activation sum is needed.  Blocks sit at 2-byte aligned
// LDS offsets: 16-byte pieces are read as aligned dwords and shifted.
//
// The activations are copied in the order the lanes read them, with
// dword copies (global_load_lds_dword) whose lanes gather from the Q8_1
// blocks: for k = 0 .. 3, unit n's 16 values at X_k + 16n, and the four f16
// block scales (with the pad beside each) at DX + 16n.  Each read is then
// one 16-byte LDS load by consecutive lanes at consecutive addresses; read in
// place from the raw 40-byte blocks, the four dwords of every unit fell in 8
// of the 32 banks and took twice as long.  sc * D is an integer product
// (|D| <= 16 * 32 * 127) and the f16 scales enter the fma directly.
constexpr int kQ6T1Rounds = 8;     // 1 KB copies per wave (its LDS region)
constexpr int kQ6T1ABlocks = 38;   // super-blocks always inside the copies
constexpr int kQ6T1MaxBlocks = 46; // + at most 8 in registers (2 chunks per lane)

// Weight copies issued before the workgroup's activation barrier; the rest
// follow it.  Issuing all of them first let the CU's first workgroup take
// all its bytes before the second got any, leaving the second's whole
// compute after the last arrival.
constexpr int kQ6T1Early = 5;

// Activation bytes of a row of nb super-blocks in unit order: G groups of 16
// units, five 256-byte copies per group (X_0 .. X_3, DX).
__host__ __device__ constexpr int q6t1_groups(int nb) { return (nb + 3) / 4; }
__host__ __device__ constexpr int q6t1_act_bytes(int nb) { return 5 * 256 * q6t1_groups(nb); }

// 16 (8) bytes that start sh bytes past the dword-aligned LDS address a (the
// fifth (third) dword read is inside the LDS allocation: every caller's piece
// ends at least 4 bytes before the end of its block or region).
__device__ __forceinline__ uint4 lds16_sh(const uint32_t* a, uint32_t sh) {
  const uint32_t w0 = a[0], w1 = a[1], w2 = a[2], w3 = a[3], w4 = a[4];
  return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh),
                    __builtin_amdgcn_alignbyte(w3, w2, sh), __builtin_amdgcn_alignbyte(w4, w3, sh));
}
__device__ __forceinline__ uint2 lds8_sh(const uint32_t* a, uint32_t sh) {
  const uint32_t w0 = a[0], w1 = a[1], w2 = a[2];
  return make_uint2(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh));
}

// Workgroup blk of the one-token Q6_K matvec (rows 8 blk .. 8 blk + 7), with
// the workgroup's LDS at lds.
template <bool DEBUG>
__device__ __forceinline__ void q6k_t1_body(uint8_t* lds, int blk, const uint8_t* w, const uint8_t* xq,
                                            float* __restrict__ y, int M, int nb, int32_t* __restrict__ dbgD) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_raw = blk * kMmvqWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves read a valid row, store nothing
  const size_t row_off = static_cast<size_t>(row) * nb * kQ6Bytes;
  const int shift = static_cast<int>(row_off & 15u);
  const uint8_t* a0 = w + (row_off - shift);                          // 16-byte aligned
  const int nch = (shift + nb * kQ6Bytes + 15) >> 4;                   // aligned chunks covering the row
  const int cb0 = (shift + kQ6T1ABlocks * kQ6Bytes) >> 4;              // first chunk held in registers
  const int G = q6t1_groups(nb);
  constexpr int kG = q6t1_groups(kQ6T1MaxBlocks);  // layout stride fixed: LDS offsets are immediates
  uint8_t* wl = lds + wave * kQ6T1Rounds * 1024;                       // this wave's region
  const uint8_t* xl = lds + kMmvqWaves * kQ6T1Rounds * 1024;           // activations in unit order
  const uint32_t wl_a = lds_addr(wl), xl_a = lds_addr(xl);
  // 1. the activations: group g (units 16g .. 16g + 15) by wave g % 8; lane l
  //    carries dword l % 4 of unit 16g + l / 4 (units past the row repeat the last)
  for (int g = wave; g < G; g += kMmvqWaves) {
    const int nc = min(16 * g + (lane >> 2), 4 * nb - 1);
    const uint8_t* src = xq + (8 * (nc >> 2) + 4 * ((nc >> 1) & 1)) * kQ8Bytes;  // block 8b + 4h
#pragma unroll
    for (int k = 0; k < 4; ++k) dma4(src + k * kQ8Bytes + 4 + 16 * (nc & 1) + 4 * (lane & 3), xl_a + 256 * (kG * k + g));
    dma4(src + (lane & 3) * kQ8Bytes, xl_a + 256 * (4 * kG + g));  // block 8b + 4h + l % 4: f16 d + pad
  }
  // 2. the first copies of the row into the region (chunks past the row re-read its last one)
#pragma unroll
  for (int r = 0; r < kQ6T1Early; ++r) dma16<true>(a0 + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
  // 3. this wave's activation copies (issued first) are done; then everyone's
  wait_vmcnt<kQ6T1Early>();
  __syncthreads();
  // 4. the rest of the row: the remaining copies, then chunks cb0 .. cb0 + 127
  //    into registers (clamped the same way)
#pragma unroll
  for (int r = kQ6T1Early; r < kQ6T1Rounds; ++r) dma16<true>(a0 + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
  const uint4 rb0 = ld16_nt(a0 + 16 * min(cb0 + lane, nch - 1));
  const uint4 rb1 = ld16_nt(a0 + 16 * min(cb0 + 64 + lane, nch - 1));
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    // copies holding super-blocks 16u .. 16u + 15 (at most shift + 32 * 210 < 7 KB for u = 1)
    if (u == 0) wait_vmcnt<4 + 2>();
    else if (u == 1) wait_vmcnt<1 + 2>();
    else {
      // the register chunks over super-blocks 0 .. 9 of the region (this wave's reads of them are done)
      *reinterpret_cast<uint4*>(wl + 16 * lane) = rb0;
      *reinterpret_cast<uint4*>(wl + 1024 + 16 * lane) = rb1;
      wait_vmcnt<0>();
    }
    const int n = 64 * u + lane, b = n >> 2, h = (n >> 1) & 1, q = n & 1;
    if (b < nb) {
      const int vb = shift + b * kQ6Bytes;
      const uint8_t* blk = wl + (b < kQ6T1ABlocks ? vb : vb - 16 * cb0);
      // every piece sits a multiple of 4 bytes into the block: one shift for all
      const uint32_t sh = static_cast<uint32_t>(vb) & 3u;
      const uint32_t* ba = reinterpret_cast<const uint32_t*>(blk - sh);
      const uint4 pa = lds16_sh(ba + 16 * h + 4 * q, sh);      // ql[64h + 16q ..]: k = 0 (low), 2 (high nibbles)
      const uint4 pb = lds16_sh(ba + 16 * h + 8 + 4 * q, sh);  // ql[64h + 32 + 16q ..]: k = 1 and 3
      const uint4 ph = lds16_sh(ba + 32 + 8 * h + 4 * q, sh);  // qh[32h + 16q ..]: bits 2k, 2k + 1
      const uint2 sc8 = lds8_sh(ba + 48 + 2 * h, sh);          // sc[8h .. 8h + 7]: k's scale is byte 2k + q
      const uint32_t scx = sc8.x >> (8 * q), scy = sc8.y >> (8 * q);
      const uint4 dxw = *reinterpret_cast<const uint4*>(xl + 256 * 4 * kG + 16 * n);
      const uint32_t dx[4] = {dxw.x, dxw.y, dxw.z, dxw.w};
      const uint32_t qa[4] = {pa.x, pa.y, pa.z, pa.w}, qb[4] = {pb.x, pb.y, pb.z, pb.w};
      const uint32_t qh[4] = {ph.x, ph.y, ph.z, ph.w};
      float accu = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // half q of Q8_1 block 8b + 4h + k
        const uint4 xw = *reinterpret_cast<const uint4*>(xl + 256 * kG * k + 16 * n);
        const uint32_t xv[4] = {xw.x, xw.y, xw.z, xw.w};
        int D = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = ((k & 1) ? qb[i] : qa[i]) >> ((k >> 1) * 4);
          const uint32_t hi = (qh[i] >> (2 * k)) & 0x03030303u;
          const uint32_t v = (lo & 0x0f0f0f0fu) | __builtin_amdgcn_perm(kQ6HiTable, kQ6HiTable, hi);
          D = i == 0 ? dot4_0(v, xv[0]) : dot4(v, xv[i], D);
        }
        const int sc = static_cast<int8_t>(((k < 2) ? scx : scy) >> (16 * (k & 1)));
        if constexpr (DEBUG) {
          if (row_ok) dbgD[static_cast<size_t>(row) * (nb * 16) + 16 * b + 8 * h + 2 * k + q] = D;
        } else {
          accu = fmaf(h2f(dx[k]), static_cast<float>(__mul24(sc, D)), accu);
        }
      }
      if constexpr (!DEBUG) acc = fmaf(h2f(*reinterpret_cast<const uint16_t*>(blk + 208)), accu, acc);
    }
  }
  wait_vmcnt<0>();
  if constexpr (!DEBUG) {
    const float s = wave_sum(acc);
    if (lane == 0 && row_ok) y[row] = s;
  }
}

template <bool DEBUG>
__global__ __launch_bounds__(kMmvqThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_q6k_t1_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb,
                        int32_t* __restrict__ dbgD) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  q6k_t1_body<DEBUG>(lds, blockIdx.x, w, xq, y, M, nb, dbgD);
}

constexpr size_t kQ6T1Lds = static_cast<size_t>(kMmvqWaves) * kQ6T1Rounds * 1024 + q6t1_act_bytes(kQ6T1MaxBlocks);

// Whether the one-token Q6_K kernel takes the shape: rows of at most 46
// super-blocks, and a matrix that ends on a 16-byte boundary (its aligned
// chunk reads then stay inside the matrix).
static bool q6k_t1_fits(int M, int nb) {
  return nb <= kQ6T1MaxBlocks && (static_cast<int64_t>(M) * nb) % 8 == 0;
}

template <bool DEBUG>
static int launch_mmvq_q6k_t1(const void* w, const void* xq, float* y, int M, int nb, int32_t* D, hipStream_t st) {
  const size_t lds = kQ6T1Lds;
  static bool attr_set = false;
  if (!attr_set) {
    const size_t lmax = lds;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_q6k_t1_kernel<DEBUG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lmax)) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((M + kMmvqWaves - 1) / kMmvqWaves), block(kMmvqThreads);
  hipLaunchKernelGGL((mmvq_q6k_t1_kernel<DEBUG>), grid, block, lds, st, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), y, M, nb, D);
  return launch_status();
}

// Two to four tokens, Q6_K: the one-token Q6_K design with one 16-wave
// workgroup per CU, so the T tokens' activations (gathered in unit order,
// 14 KB per token at K = 11008) are copied once per CU.  To fit them beside
// sixteen rows, a wave copies the first 6 KB of its row (super-blocks 0 .. 28
// for any shift) into its LDS region and loads the rest (at most 14 more
// super-blocks) as three 16-byte register chunks per lane, written over the
// region's first 3 KB once unit round 0 (super-blocks 0 .. 15) is done.  Each
// lane forms its unit's 64 signed values once and multiplies them with every
// token.
constexpr int kQ6TnWaves = 16;
constexpr int kQ6TnRounds = 6;      // 1 KB copies per wave (its LDS region)
constexpr int kQ6TnEarly = 3;       // of them issued before the activation barrier (measured 3 .. 6)
constexpr int kQ6TnABlocks = 29;    // super-blocks always inside the copies
constexpr int kQ6TnMaxBlocks = 43;  // + at most 14 in the register chunks
static_assert(kQ6TnWaves * kQ6TnRounds * 1024 + 4 * q6t1_act_bytes(kQ6TnMaxBlocks) <= 160 * 1024,
              "sixteen row regions and four tokens");

template <int T, bool DEBUG>
__global__ __launch_bounds__(64 * kQ6TnWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_q6k_tn_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb,
                        int32_t* __restrict__ dbgD) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_raw = blockIdx.x * kQ6TnWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves read a valid row, store nothing
  const size_t row_off = static_cast<size_t>(row) * nb * kQ6Bytes;
  const int shift = static_cast<int>(row_off & 15u);
  const uint8_t* a0 = w + (row_off - shift);                          // 16-byte aligned
  const int nch = (shift + nb * kQ6Bytes + 15) >> 4;                   // aligned chunks covering the row
  const int cb0 = (shift + kQ6TnABlocks * kQ6Bytes) >> 4;              // first chunk held in registers
  const int G = q6t1_groups(nb);
  // layout strides fixed at the largest row, so every LDS offset below is an immediate
  constexpr int kG = q6t1_groups(kQ6TnMaxBlocks), tb = q6t1_act_bytes(kQ6TnMaxBlocks);
  uint8_t* wl = lds + wave * kQ6TnRounds * 1024;                       // this wave's region
  const uint8_t* xl = lds + kQ6TnWaves * kQ6TnRounds * 1024;           // activations in unit order
  const uint32_t wl_a = lds_addr(wl), xl_a = lds_addr(xl);
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  // 1. the activations of token t, group g (units 16g .. 16g + 15), pair c = t * G + g by
  //    wave c % 16: the layout of the one-token kernel, token t at xl + t * tb
  for (int c = wave; c < T * G; c += kQ6TnWaves) {
    const int t = c / G, g = c - t * G;
    const int nc = min(16 * g + (lane >> 2), 4 * nb - 1);
    const uint8_t* src = xq + t * xstride + (8 * (nc >> 2) + 4 * ((nc >> 1) & 1)) * kQ8Bytes;
    const uint32_t dst = xl_a + t * tb;
#pragma unroll
    for (int k = 0; k < 4; ++k) dma4(src + k * kQ8Bytes + 4 + 16 * (nc & 1) + 4 * (lane & 3), dst + 256 * (kG * k + g));
    dma4(src + (lane & 3) * kQ8Bytes, dst + 256 * (4 * kG + g));
  }
  // 2. the first copies of the row (chunks past the row re-read its last one)
#pragma unroll
  for (int r = 0; r < kQ6TnEarly; ++r) dma16<true>(a0 + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
  // 3. this wave's activation copies (issued first) are done; then everyone's;
  //    then the rest of the row and the register chunks
  wait_vmcnt<kQ6TnEarly>();
  __syncthreads();
#pragma unroll
  for (int r = kQ6TnEarly; r < kQ6TnRounds; ++r) dma16<true>(a0 + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
  uint4 rb[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) rb[j] = ld16_nt(a0 + 16 * min(cb0 + 64 * j + lane, nch - 1));
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    if (u == 0) {
      // copies holding super-blocks 0 .. 15 (shift + 16 * 210 < 4 KB)
      wait_vmcnt<kQ6TnRounds - 4 + 3>();
    } else if (u == 1) {
      // the register chunks over super-blocks 0 .. 14 of the region (this wave's reads of them are done);
      // the copies are older than the register loads, so they are done too
#pragma unroll
      for (int j = 0; j < 3; ++j) *reinterpret_cast<uint4*>(wl + 1024 * j + 16 * lane) = rb[j];
      wait_vmcnt<0>();
    }
    const int n = 64 * u + lane, b = n >> 2, h = (n >> 1) & 1, q = n & 1;
    if (b < nb) {
      const int vb = shift + b * kQ6Bytes;
      const uint8_t* blk = wl + (b < kQ6TnABlocks ? vb : vb - 16 * cb0);
      const uint32_t sh = static_cast<uint32_t>(vb) & 3u;
      const uint32_t* ba = reinterpret_cast<const uint32_t*>(blk - sh);
      const uint4 pa = lds16_sh(ba + 16 * h + 4 * q, sh);      // ql[64h + 16q ..]: k = 0 (low), 2 (high nibbles)
      const uint4 pb = lds16_sh(ba + 16 * h + 8 + 4 * q, sh);  // ql[64h + 32 + 16q ..]: k = 1 and 3
      const uint4 ph = lds16_sh(ba + 32 + 8 * h + 4 * q, sh);  // qh[32h + 16q ..]: bits 2k, 2k + 1
      const uint2 sc8 = lds8_sh(ba + 48 + 2 * h, sh);          // sc[8h .. 8h + 7]: k's scale is byte 2k + q
      const uint32_t scx = sc8.x >> (8 * q), scy = sc8.y >> (8 * q);
      const float d = h2f(*reinterpret_cast<const uint16_t*>(blk + 208));
      const uint32_t qa[4] = {pa.x, pa.y, pa.z, pa.w}, qb[4] = {pb.x, pb.y, pb.z, pb.w};
      const uint32_t qh[4] = {ph.x, ph.y, ph.z, ph.w};
      uint32_t v[4][4];  // signed values q6 - 32 of k = 0 .. 3
      int sc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = ((k & 1) ? qb[i] : qa[i]) >> ((k >> 1) * 4);
          const uint32_t hi = (qh[i] >> (2 * k)) & 0x03030303u;
          v[k][i] = (lo & 0x0f0f0f0fu) | __builtin_amdgcn_perm(kQ6HiTable, kQ6HiTable, hi);
        }
        sc[k] = static_cast<int8_t>(((k < 2) ? scx : scy) >> (16 * (k & 1)));
      }
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint8_t* xt = xl + t * tb;
        const uint4 dxw = *reinterpret_cast<const uint4*>(xt + 256 * 4 * kG + 16 * n);
        const uint32_t dx[4] = {dxw.x, dxw.y, dxw.z, dxw.w};
        float accu = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // half q of Q8_1 block 8b + 4h + k of token t
          const uint4 xw = *reinterpret_cast<const uint4*>(xt + 256 * kG * k + 16 * n);
          int D = dot4_0(v[k][0], xw.x);
          D = dot4(v[k][1], xw.y, D);
          D = dot4(v[k][2], xw.z, D);
          D = dot4(v[k][3], xw.w, D);
          if constexpr (DEBUG) {
            if (row_ok) dbgD[(static_cast<size_t>(t) * M + row) * (nb * 16) + 16 * b + 8 * h + 2 * k + q] = D;
          } else {
            accu = fmaf(h2f(dx[k]), static_cast<float>(__mul24(sc[k], D)), accu);
          }
        }
        if constexpr (!DEBUG) acc[t] = fmaf(d, accu, acc[t]);
      }
    }
  }
  wait_vmcnt<0>();
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && row_ok) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

template <int T, bool DEBUG>
static int launch_mmvq_q6k_tn(const void* w, const void* xq, float* y, int M, int nb, int32_t* D, hipStream_t st) {
  const size_t lds = static_cast<size_t>(kQ6TnWaves) * kQ6TnRounds * 1024 +
                     static_cast<size_t>(T) * q6t1_act_bytes(kQ6TnMaxBlocks);
  static bool attr_set = false;
  if (!attr_set) {
    const size_t lmax = lds;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_q6k_tn_kernel<T, DEBUG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lmax)) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((M + kQ6TnWaves - 1) / kQ6TnWaves), block(64 * kQ6TnWaves);
  hipLaunchKernelGGL((mmvq_q6k_tn_kernel<T, DEBUG>), grid, block, lds, st, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), y, M, nb, D);
  return launch_status();
}

// Five to eight tokens, Q6_K: the same 16-row workgroups with the row in
// segments of at most 22 super-blocks (two at K = 11008), so the T tokens'
// activations of a segment fit beside sixteen row segments.  A wave copies
// the 16-byte aligned chunks that cover its row segment (at most 5 KB) into
// its LDS region, after the workgroup's gather of the segment's
// activations; each segment ends with every copy landed and a barrier
// before the region is reused.
constexpr int kQ6TsRounds = 5;     // 1 KB copies per wave per segment
constexpr int kQ6TsMaxBlocks = 22; // super-blocks per segment (22 * 210 + 15 <= 5 KB)

template <int T>
static int q6ts_seg_blocks(int nb) {
  constexpr int kBudget = 160 * 1024 - kQ6TnWaves * kQ6TsRounds * 1024;  // activation bytes
  int cb = kQ6TsMaxBlocks;
  while (cb > 4 && T * q6t1_act_bytes(cb) > kBudget) --cb;
  const int nseg = (nb + cb - 1) / cb;
  return (nb + nseg - 1) / nseg;
}

template <int T, bool DEBUG>
__global__ __launch_bounds__(64 * kQ6TnWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_q6k_ts_kernel(const uint8_t* w, const uint8_t* xq, float* __restrict__ y, int M, int nb, int cb,
                        int32_t* __restrict__ dbgD) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row_raw = blockIdx.x * kQ6TnWaves + wave;
  const bool row_ok = row_raw < M;
  const int row = row_ok ? row_raw : M - 1;  // out-of-range waves read a valid row, store nothing
  const size_t row_off = static_cast<size_t>(row) * nb * kQ6Bytes;
  const int tb = q6t1_act_bytes(cb);                                   // activation bytes per token
  const int Gs = q6t1_groups(cb);                                      // layout stride (groups)
  uint8_t* wl = lds + wave * kQ6TsRounds * 1024;                       // this wave's region
  const uint8_t* xl = lds + kQ6TnWaves * kQ6TsRounds * 1024;           // activations in unit order
  const uint32_t wl_a = lds_addr(wl), xl_a = lds_addr(xl);
  const size_t xstride = static_cast<size_t>(nb) * 8 * kQ8Bytes;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  for (int b0 = 0; b0 < nb; b0 += cb) {
    const int nbc = min(cb, nb - b0);
    const int G = q6t1_groups(nbc);
    if (b0 > 0) __syncthreads();  // every wave is done with the previous segment
    // 1. the segment's activations, token t at xl + t * tb (groups of 16 units)
    for (int c = wave; c < T * G; c += kQ6TnWaves) {
      const int t = c / G, g = c - t * G;
      const int nc = min(16 * g + (lane >> 2), 4 * nbc - 1);
      const uint8_t* src = xq + t * xstride + (8 * (b0 + (nc >> 2)) + 4 * ((nc >> 1) & 1)) * kQ8Bytes;
      const uint32_t dst = xl_a + t * tb;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dma4(src + k * kQ8Bytes + 4 + 16 * (nc & 1) + 4 * (lane & 3), dst + 256 * (Gs * k + g));
      dma4(src + (lane & 3) * kQ8Bytes, dst + 256 * (4 * Gs + g));
    }
    // 2. the chunks covering the row segment (chunks past it re-read its last one)
    const size_t seg_off = row_off + static_cast<size_t>(b0) * kQ6Bytes;
    const int shift = static_cast<int>(seg_off & 15u);
    const uint8_t* a0 = w + (seg_off - shift);
    const int nch = (shift + nbc * kQ6Bytes + 15) >> 4;
#pragma unroll
    for (int r = 0; r < kQ6TsRounds; ++r) dma16<true>(a0 + 16 * min(64 * r + lane, nch - 1), wl_a + 1024 * r);
    // 3. this wave's activation copies (issued first) are done; then everyone's
    wait_vmcnt<kQ6TsRounds>();
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // copies holding super-blocks 16u .. 16u + 15 (shift + 16 * 210 < 4 KB)
      if (u == 0) wait_vmcnt<1>();
      else wait_vmcnt<0>();
      const int n = 64 * u + lane, b = n >> 2, h = (n >> 1) & 1, q = n & 1;
      if (b < nbc) {
        const int vb = shift + b * kQ6Bytes;
        const uint8_t* blk = wl + vb;
        const uint32_t sh = static_cast<uint32_t>(vb) & 3u;
        const uint32_t* ba = reinterpret_cast<const uint32_t*>(blk - sh);
        const uint4 pa = lds16_sh(ba + 16 * h + 4 * q, sh);      // ql[64h + 16q ..]: k = 0 (low), 2 (high nibbles)
        const uint4 pb = lds16_sh(ba + 16 * h + 8 + 4 * q, sh);  // ql[64h + 32 + 16q ..]: k = 1 and 3
        const uint4 ph = lds16_sh(ba + 32 + 8 * h + 4 * q, sh);  // qh[32h + 16q ..]: bits 2k, 2k + 1
        const uint2 sc8 = lds8_sh(ba + 48 + 2 * h, sh);          // sc[8h .. 8h + 7]: k's scale is byte 2k + q
        const uint32_t scx = sc8.x >> (8 * q), scy = sc8.y >> (8 * q);
        const float d = h2f(*reinterpret_cast<const uint16_t*>(blk + 208));
        const uint32_t qa[4] = {pa.x, pa.y, pa.z, pa.w}, qb[4] = {pb.x, pb.y, pb.z, pb.w};
        const uint32_t qh[4] = {ph.x, ph.y, ph.z, ph.w};
        uint32_t v[4][4];  // signed values q6 - 32 of k = 0 .. 3
        int sc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = ((k & 1) ? qb[i] : qa[i]) >> ((k >> 1) * 4);
            const uint32_t hi = (qh[i] >> (2 * k)) & 0x03030303u;
            v[k][i] = (lo & 0x0f0f0f0fu) | __builtin_amdgcn_perm(kQ6HiTable, kQ6HiTable, hi);
          }
          sc[k] = static_cast<int8_t>(((k < 2) ? scx : scy) >> (16 * (k & 1)));
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint8_t* xt = xl + t * tb;
          const uint4 dxw = *reinterpret_cast<const uint4*>(xt + 256 * 4 * Gs + 16 * n);
          const uint32_t dx[4] = {dxw.x, dxw.y, dxw.z, dxw.w};
          float accu = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint4 xw = *reinterpret_cast<const uint4*>(xt + 256 * Gs * k + 16 * n);
            int D = dot4_0(v[k][0], xw.x);
            D = dot4(v[k][1], xw.y, D);
            D = dot4(v[k][2], xw.z, D);
            D = dot4(v[k][3], xw.w, D);
            if constexpr (DEBUG) {
              if (row_ok)
                dbgD[(static_cast<size_t>(t) * M + row) * (nb * 16) + 16 * (b0 + b) + 8 * h + 2 * k + q] = D;
            } else {
              accu = fmaf(h2f(dx[k]), static_cast<float>(__mul24(sc[k], D)), accu);
            }
          }
          if constexpr (!DEBUG) acc[t] = fmaf(d, accu, acc[t]);
        }
      }
    }
    wait_vmcnt<0>();
  }
  if constexpr (!DEBUG) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && row_ok) y[static_cast<size_t>(t) * M + row] = s;
    }
  }
}

template <int T, bool DEBUG>
static int launch_mmvq_q6k_ts(const void* w, const void* xq, float* y, int M, int nb, int32_t* D, hipStream_t st) {
  const int cb = q6ts_seg_blocks<T>(nb);
  const size_t lds = static_cast<size_t>(kQ6TnWaves) * kQ6TsRounds * 1024 + static_cast<size_t>(T) * q6t1_act_bytes(cb);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_q6k_ts_kernel<T, DEBUG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const dim3 grid((M + kQ6TnWaves - 1) / kQ6TnWaves), block(64 * kQ6TnWaves);
  hipLaunchKernelGGL((mmvq_q6k_ts_kernel<T, DEBUG>), grid, block, lds, st, static_cast<const uint8_t*>(w),
                     static_cast<const uint8_t*>(xq), y, M, nb, cb, D);
  return launch_status();
}

// Q6_K segments: at most 4 * q6_rounds(T) blocks (the pieces held in
// registers) and kQ6ActBudget bytes of staged activations (with the waves'
// piece regions two workgroups fit a CU); the row is split into segments
// of equal length.
constexpr int kQ6ActBudget = 44 * 1024;
template <bool DEBUG>
static int launch_mmvq_q6k(const void* w, const void* xq, float* y, int M, int nb, int T,
                           int32_t* D, hipStream_t st, const SlotArgs* slots = nullptr, int nslots = 0) {
  // one token: the LDS-copy kernel where it takes the shape
  if (!slots && T == 1 && q6k_t1_fits(M, nb)) return launch_mmvq_q6k_t1<DEBUG>(w, xq, y, M, nb, D, st);
  if (!slots && T >= 2 && T <= 4 && nb <= kQ6TnMaxBlocks && (static_cast<int64_t>(M) * nb) % 8 == 0) {
    if (T == 2) return launch_mmvq_q6k_tn<2, DEBUG>(w, xq, y, M, nb, D, st);
    if (T == 3) return launch_mmvq_q6k_tn<3, DEBUG>(w, xq, y, M, nb, D, st);
    return launch_mmvq_q6k_tn<4, DEBUG>(w, xq, y, M, nb, D, st);
  }
  if (!slots && T >= 5 && T <= 8 && (static_cast<int64_t>(M) * nb) % 8 == 0) {
    if (T == 5) return launch_mmvq_q6k_ts<5, DEBUG>(w, xq, y, M, nb, D, st);
    if (T == 6) return launch_mmvq_q6k_ts<6, DEBUG>(w, xq, y, M, nb, D, st);
    if (T == 7) return launch_mmvq_q6k_ts<7, DEBUG>(w, xq, y, M, nb, D, st);
    return launch_mmvq_q6k_ts<8, DEBUG>(w, xq, y, M, nb, D, st);
  }
  const SlotArgs SA = slots ? *slots : SlotArgs{};
  int cmax = kQ6ActBudget / (T * kQK * 3 / 2);
  if (cmax > 4 * q6_rounds(T)) cmax = 4 * q6_rounds(T);
  if (cmax < 1) cmax = 1;
  const int nseg = (nb + cmax - 1) / cmax;
  const int cb = (nb + nseg - 1) / nseg;
  const dim3 grid((M + kMmvqWaves - 1) / kMmvqWaves), block(kMmvqThreads);
  const size_t lds = mmvq_lds_bytes(T, cb) + static_cast<size_t>(kMmvqWaves) * kQ6WaveRegion;
  const uint8_t* wp = static_cast<const uint8_t*>(w);
  const uint8_t* xp = static_cast<const uint8_t*>(xq);
  if (slots) {
    if (DEBUG || T != 1) return QMM_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((mmvq_q6k_kernel<1, false, true>), dim3(grid.x, nslots), block, lds, st, wp, xp, y, M, nb,
                       cb, D, SA);
    return launch_status();
  }
  switch (T) {
#define QMM_CASE(TT) \
  case TT: hipLaunchKernelGGL((mmvq_q6k_kernel<TT, DEBUG>), grid, block, lds, st, wp, xp, y, M, nb, cb, D, SA); break;
    QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
    default: return QMM_ERR_SHAPE;
  }
  return launch_status();
}

// Host checks shared by the three formats.
static int check_mmvq(const void* w, const void* xq, const float* y, int64_t M, int64_t K, int64_t T) {
  if (M < 1 || K < kQK || (K % kQK) != 0 || T < 1 || T > QMM_MMVQ_MAX_T) return QMM_ERR_SHAPE;
  if (M > 0x7fffffff || K / kQK > (1 << 20)) return QMM_ERR_SHAPE;
  if (!w || !xq || !y) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(y)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

// Two one-token matvecs on one activation row in one launch (say the two
// weight matrices that read the same normalised hidden state in a decode
// step): workgroups 0 .. na - 1 run matrix a, the rest matrix b, each with
// the workgroup code of its own one-token kernel, so each output has the
// bits that kernel gives.  The matrix with more bytes per row goes first,
// since workgroups start in index order: the lighter workgroups then fill
// the CUs as the heavier ones finish, and the launch ends with one tail
// instead of two.
struct PairSide {
  const uint8_t* w;
  float* y;
  int M, nblk, cb;
};

template <int FMT>
__device__ __forceinline__ void t1_body(uint8_t* lds, int blk, const PairSide& S, const uint8_t* xq, int nb) {
  if constexpr (FMT == QMM_Q6_K)
    q6k_t1_body<false>(lds, blk, S.w, xq, S.y, S.M, nb, nullptr);
  else
    q45_t1_body<FMT, false>(lds, blk, S.w, xq, S.y, S.M, nb, S.cb, nullptr, nullptr);
}

template <int FA, int FB>
__global__ __launch_bounds__(kMmvqThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void mmvq_pair_t1_kernel(PairSide A, PairSide B, const uint8_t* xq, int nb) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int blk = blockIdx.x;
  if (blk < A.nblk)  // uniform per workgroup
    t1_body<FA>(lds, blk, A, xq, nb);
  else
    t1_body<FB>(lds, blk - A.nblk, B, xq, nb);
}

template <int FMT>
static size_t pair_lds_bytes(int cb) {
  if constexpr (FMT == QMM_Q6_K) return kQ6T1Lds;
  else return t1_lds_bytes<FMT>(cb);
}
template <int FMT>
static size_t pair_lds_max() {
  if constexpr (FMT == QMM_Q6_K) return kQ6T1Lds;
  else return t1_lds_bytes<FMT>(MvDma<FMT>::kMaxBlocks);
}

template <int FA, int FB>
static int launch_pair(const PairSide& A, const PairSide& B, const void* xq, int nb, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    const size_t lmax = std::max(pair_lds_max<FA>(), pair_lds_max<FB>());
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&mmvq_pair_t1_kernel<FA, FB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lmax)) != hipSuccess)
      return QMM_ERR_HIP;
    attr_set = true;
  }
  const size_t lds = std::max(pair_lds_bytes<FA>(A.cb), pair_lds_bytes<FB>(B.cb));
  hipLaunchKernelGGL((mmvq_pair_t1_kernel<FA, FB>), dim3(A.nblk + B.nblk), dim3(kMmvqThreads), lds, st, A, B,
                     static_cast<const uint8_t*>(xq), nb);
  return launch_status();
}

template <int FA>
static int launch_pair_b(int fb, const PairSide& A, const PairSide& B, const void* xq, int nb, hipStream_t st) {
  if (fb == QMM_Q4_K) return launch_pair<FA, QMM_Q4_K>(A, B, xq, nb, st);
  if (fb == QMM_Q5_K) return launch_pair<FA, QMM_Q5_K>(A, B, xq, nb, st);
  return launch_pair<FA, QMM_Q6_K>(A, B, xq, nb, st);
}

static int row_block_bytes(int fmt) { return fmt == QMM_Q4_K ? kQ4Bytes : fmt == QMM_Q5_K ? kQ5Bytes : kQ6Bytes; }

static int seg_blocks_t1(int fmt, int nb) {
  if (fmt == QMM_Q4_K) return t1_seg_blocks<QMM_Q4_K>(nb);
  if (fmt == QMM_Q5_K) return t1_seg_blocks<QMM_Q5_K>(nb);
  return nb;
}

static int mmvq_one(int fmt, const void* w, const void* xq, float* y, int M, int nb, hipStream_t st) {
  if (fmt == QMM_Q4_K) return launch_mmvq_q4k<false>(w, xq, y, M, nb, 1, nullptr, nullptr, st);
  if (fmt == QMM_Q5_K) return launch_mmvq_q4k<false, QMM_Q5_K>(w, xq, y, M, nb, 1, nullptr, nullptr, st);
  return launch_mmvq_q6k<false>(w, xq, y, M, nb, 1, nullptr, st);
}

int mmvq_pair_launch(int fa, const void* wa, int Ma, float* ya, int fb, const void* wb, int Mb, float* yb,
                     const void* xq, int nb, hipStream_t st) {
  // one launch only where both one-token kernels take their shapes;
  // otherwise the two matvecs one after the other
  if ((fa == QMM_Q6_K && !q6k_t1_fits(Ma, nb)) || (fb == QMM_Q6_K && !q6k_t1_fits(Mb, nb))) {
    const int r = mmvq_one(fa, wa, xq, ya, Ma, nb, st);
    return r != QMM_OK ? r : mmvq_one(fb, wb, xq, yb, Mb, nb, st);
  }
  if (row_block_bytes(fb) > row_block_bytes(fa)) {
    std::swap(fa, fb);
    std::swap(wa, wb);
    std::swap(Ma, Mb);
    std::swap(ya, yb);
  }
  const PairSide A{static_cast<const uint8_t*>(wa), ya, Ma, (Ma + kMmvqWaves - 1) / kMmvqWaves, seg_blocks_t1(fa, nb)};
  const PairSide B{static_cast<const uint8_t*>(wb), yb, Mb, (Mb + kMmvqWaves - 1) / kMmvqWaves, seg_blocks_t1(fb, nb)};
  if (fa == QMM_Q4_K) return launch_pair_b<QMM_Q4_K>(fb, A, B, xq, nb, st);
  if (fa == QMM_Q5_K) return launch_pair_b<QMM_Q5_K>(fb, A, B, xq, nb, st);
  return launch_pair_b<QMM_Q6_K>(fb, A, B, xq, nb, st);
}

int debug_mmvq(int fmt, const void* w, const void* xq, int32_t* D, int32_t* S, int64_t M,
               int64_t K, int64_t T, hipStream_t st) {
  if (fmt == QMM_Q4_K)
    return launch_mmvq_q4k<true>(w, xq, nullptr, static_cast<int>(M), static_cast<int>(K / kQK),
                                 static_cast<int>(T), D, S, st);
  if (fmt == QMM_Q5_K)
    return launch_mmvq_q4k<true, QMM_Q5_K>(w, xq, nullptr, static_cast<int>(M), static_cast<int>(K / kQK),
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

extern "C" int mmvq_q5k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                        void* stream) {
  const int st = check_mmvq(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  return launch_mmvq_q4k<false, QMM_Q5_K>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK),
                                          static_cast<int>(T), nullptr, nullptr, to_stream(stream));
}

extern "C" int mmvq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                        void* stream) {
  const int st = check_mmvq(w, xq, y, M, K, T);
  if (st != QMM_OK) return st;
  return launch_mmvq_q6k<false>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK),
                                static_cast<int>(T), nullptr, to_stream(stream));
}

extern "C" int mmvq_pair(int fmt_a, const void* wa, int64_t Ma, float* ya, int fmt_b, const void* wb, int64_t Mb,
                         float* yb, const void* xq, int64_t K, void* stream) {
  for (int f : {fmt_a, fmt_b})
    if (f != QMM_Q4_K && f != QMM_Q5_K && f != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  int st = check_mmvq(wa, xq, ya, Ma, K, 1);
  if (st != QMM_OK) return st;
  st = check_mmvq(wb, xq, yb, Mb, K, 1);
  if (st != QMM_OK) return st;
  if (Ma + Mb > 0x7fffffff) return QMM_ERR_SHAPE;
  return mmvq_pair_launch(fmt_a, wa, static_cast<int>(Ma), ya, fmt_b, wb, static_cast<int>(Mb), yb, xq,
                          static_cast<int>(K / kQK), to_stream(stream));
}

extern "C" int moe_slot_mmvq(int fmt, const void* w, int64_t E, int64_t M, int64_t K, int64_t expert_stride_bytes,
                             const void* xq, int64_t x_rows_per_token, const int32_t* ids, int64_t T,
                             int64_t top_k, float* y, void* stream) {
  if (fmt != QMM_Q4_K && fmt != QMM_Q5_K && fmt != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  if (E < 1 || E > (1 << 20) || M < 1 || M > 0x7fffffff || K < kQK || (K % kQK) != 0 || K / kQK > (1 << 20) ||
      T < 1 || top_k < 1 || top_k > E || T * top_k > 65535)
    return QMM_ERR_SHAPE;
  if (x_rows_per_token != 1 && x_rows_per_token != top_k) return QMM_ERR_SHAPE;
  const int64_t row_bytes = (K / kQK) * (fmt == QMM_Q4_K ? kQ4Bytes : fmt == QMM_Q5_K ? kQ5Bytes : kQ6Bytes);
  // Q4_K / Q5_K rows are read with aligned 16-byte loads, Q6_K rows with 2-byte aligned ones
  const int64_t stride_align = fmt == QMM_Q6_K ? 2 : 16;
  if (expert_stride_bytes < M * row_bytes || (expert_stride_bytes % stride_align) != 0) return QMM_ERR_SHAPE;
  if (!w || !xq || !ids || !y) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(ids) || !aligned16(y)) return QMM_ERR_ALIGN;
  SlotArgs S{ids, expert_stride_bytes, static_cast<int>(E), static_cast<int>(top_k),
             static_cast<int>(x_rows_per_token)};
  const int nslots = static_cast<int>(T * top_k);
  if (fmt == QMM_Q4_K)
    return launch_mmvq_q4k<false>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK), 1, nullptr, nullptr,
                                  to_stream(stream), &S, nslots);
  if (fmt == QMM_Q5_K)
    return launch_mmvq_q4k<false, QMM_Q5_K>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK), 1, nullptr,
                                            nullptr, to_stream(stream), &S, nslots);
  return launch_mmvq_q6k<false>(w, xq, y, static_cast<int>(M), static_cast<int>(K / kQK), 1, nullptr,
                                to_stream(stream), &S, nslots);
}
