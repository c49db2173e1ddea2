// MoE routed-expert grouped GEMM: route preparation, the grouped MMQ call
// and the ordered weighted combine.
//
// [GAP] lever T2 and its de-risk paragraph: the per-token expert matvec
// re-reads an expert's weights once per routed token; grouping reads them
// once per expert: (1) histogram of expert ids, prefix-sum offsets, slot ids
// scattered into per-expert buckets, (2) per-expert product on the gathered
// tokens, scatter back.  [MMQ] "MoE routing (fused gather)": the persistent
// kernel's work entries are (expert, m_tile, n_tile) and the activation rows
// are gathered through the bucket while staging.
//
// Route preparation runs in one 1024-thread workgroup (4096 slots at
// T = 512, top-8).  Buckets are stable (slots of an expert in increasing
// order) without sorting: each of the 16 waves owns a contiguous slot range;
// among 64 slots, lanes with the same expert find each other with one ballot
// per id bit, so a lane's rank among equal ids is a popcount.  Pass 1 counts
// per (wave, expert), wave scans turn counts into offsets, pass 2 repeats the
// ranking and writes every slot to its place.  It also writes the work
// prefix (m_tiles * ceil(count / 32) per expert), the column-tile prefix
// (ceil(count / 32) per expert: where each expert's repacked activation
// chunks start) and zeroes the queue counters that the grouped kernel claims
// tiles from.
//
// The combine y[t] = sum_k p[t][k] * y_slot[t*top_k + k] runs in increasing
// k with no atomics, so results are bit-reproducible.
#include "qmm_common.hpp"

#include <algorithm>

namespace qmm {

constexpr int kMoeMaxTopK = 64;
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr size_t kMoeCounterBytes = 256;
constexpr int kMoeBN = 32;   // routed tokens per tile (must match the grouped kernel)
constexpr int kMoeBM = 128;  // weight rows of the smaller grouped tile (bounds the work entries)

int mmq_moe_launch(int fmt, const uint8_t* w, int64_t stride, int M, int nb, const uint8_t* xq,
                   float* out, uint8_t* hq, unsigned* counters, const int32_t* counts, const int32_t* offsets,
                   const int32_t* bucket, const int32_t* ct_off, uint8_t* xr,
                   int max_ctiles, int E, int top_k, int rows_per_token, hipStream_t st,
                   uint8_t* xr_next = nullptr, int nb_next = 0, bool repack = true);
int64_t moe_max_ctiles(int64_t slots, int64_t E);
int moe_tile_rows(int fmt, int nb);
size_t moe_chunk_bytes(int64_t slots, int64_t E, int64_t K);

struct MoeLayout {
  unsigned* counters;
  int32_t* counts;
  int32_t* offsets;
  int32_t* ct_off;
  int32_t* bucket;
  float* scratch;
  uint8_t* chunks;
  size_t bytes;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace: counters, the route tables, the repacked routed rows and, for
// weighted calls only, the per-slot fp32 results of the ordered combine
// (last, so a per-slot call needs only the prefix).
static MoeLayout moe_layout(void* ws, int64_t M, int64_t K, int64_t T, int64_t E, int64_t top_k, bool weighted) {
  MoeLayout L{};
  uint8_t* b = static_cast<uint8_t*>(ws);
  size_t off = kMoeCounterBytes;
  const size_t ints = static_cast<size_t>(E) + 2 * static_cast<size_t>(E + 1) + static_cast<size_t>(T * top_k);
  L.counters = reinterpret_cast<unsigned*>(b);
  L.counts = reinterpret_cast<int32_t*>(b + off);
  L.offsets = L.counts + E;
  L.ct_off = L.offsets + (E + 1);
  L.bucket = L.ct_off + (E + 1);
  off = align_up(off + ints * 4, 1024);
  L.chunks = b + off;
  off = align_up(off + moe_chunk_bytes(T * top_k, E, K), 256);
  L.scratch = weighted ? reinterpret_cast<float*>(b + off) : nullptr;
  if (weighted) off += static_cast<size_t>(T * top_k) * static_cast<size_t>(M) * 4;
  L.bytes = off;
  return L;
}

size_t moe_workspace_bytes(int64_t M, int64_t K, int64_t T, int64_t E, int64_t top_k, bool weighted) {
  return moe_layout(nullptr, M, K, T, E, top_k, weighted).bytes;
}

// Fused FFN layer (moe_ffn): the down call's layout (its per-slot scratch
// last), then the gate||up call's input chunks (K = H).  The down chunks (K =
// F), written by the gate||up epilogue, sit where moe_layout puts a call's
// chunks.
struct FfnLayout {
  MoeLayout dn;
  uint8_t* chunks_gu;
  size_t bytes;
};
static FfnLayout ffn_layout(void* ws, int64_t H, int64_t F, int64_t T, int64_t E, int64_t top_k) {
  FfnLayout L{};
  L.dn = moe_layout(ws, H, F, T, E, top_k, true);
  const size_t off = align_up(L.dn.bytes, 1024);
  L.chunks_gu = static_cast<uint8_t*>(ws) + off;
  L.bytes = off + moe_chunk_bytes(T * top_k, E, H);
  return L;
}

size_t moe_ffn_workspace_bytes(int64_t H, int64_t F, int64_t T, int64_t E, int64_t top_k) {
  return ffn_layout(nullptr, H, F, T, E, top_k).bytes;
}

// Lanes of the wave holding the same expert id as this lane (v: lane
// valid): one ballot per id bit, for the ids' bits below nbits (<= 9, since
// E <= kMoeMaxE = 512; the loop has a fixed trip count so it unrolls).
__device__ __forceinline__ uint64_t peers_of(int e, bool v, int nbits) {
  uint64_t peers = __ballot(v);
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    if (b < nbits) {  // uniform
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(v && bit);
      peers &= bit ? m : ~m;
    }
  }
  return peers;
}

// Slots are ranked kRouteBatch x 64 at a time per wave; the ids of a batch
// are loaded together, so a pass costs one memory round trip per batch
// instead of one per 64 slots.
constexpr int kRouteBatch = 8;

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ ct_off, int32_t* __restrict__ bucket, unsigned* __restrict__ counters) {
  __shared__ int cnt[kRouteWaves][kMoeMaxE];
  __shared__ int s_off[kMoeMaxE + 1];
  __shared__ int s_ct[kMoeMaxE + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kRouteWaves * kMoeMaxE; i += kRouteThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int per = (n + kRouteWaves - 1) / kRouteWaves;
  const int beg = wave * per, end = min(n, beg + per);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // pass 1: per-(wave, expert) counts (LDS atomics: counts need no order)
  for (int base = beg; base < end; base += 64 * kRouteBatch) {
    int ev[kRouteBatch];
#pragma unroll
    for (int r = 0; r < kRouteBatch; ++r) {
      const int s = base + 64 * r + lane;
      ev[r] = s < end ? ids[s] : -1;
    }
#pragma unroll
    for (int r = 0; r < kRouteBatch; ++r) {
      const int e = ev[r];
      if (e >= 0 && e < E) atomicAdd(&cnt[wave][e], 1);
    }
  }
  __syncthreads();
  // exclusive prefix over waves for each expert, per-expert totals
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
    counts[e] = run;
    s_off[e] = run;
    s_ct[e] = (run + kMoeBN - 1) / kMoeBN;
  }
  __syncthreads();
  // exclusive scans over experts (E <= 512 fits one wave's 8 passes)
  if (wave == 0) {
    int off = 0, coff = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int c = e < E ? s_off[e] : 0, cv = e < E ? s_ct[e] : 0;
      // inclusive wave scans
      for (int d = 1; d < 64; d <<= 1) {
        const int cu = __shfl_up(c, d), vu = __shfl_up(cv, d);
        if (lane >= d) { c += cu; cv += vu; }
      }
      const int cx = __shfl_up(c, 1), vx = __shfl_up(cv, 1);
      const int ce = lane == 0 ? 0 : cx, ve = lane == 0 ? 0 : vx;
      if (e < E) {
        s_off[e] = off + ce;
        offsets[e] = off + ce;
        ct_off[e] = coff + ve;
      }
      off += __shfl(c, 63);
      coff += __shfl(cv, 63);
    }
    if (lane == 0) {
      offsets[E] = off;
      ct_off[E] = coff;
    }
  }
  __syncthreads();
  // pass 2: stable scatter of slot ids
  for (int base = beg; base < end; base += 64 * kRouteBatch) {
    int ev[kRouteBatch];
#pragma unroll
    for (int r = 0; r < kRouteBatch; ++r) {
      const int s = base + 64 * r + lane;
      ev[r] = s < end ? ids[s] : -1;
    }
#pragma unroll
    for (int r = 0; r < kRouteBatch; ++r) {
      if (base + 64 * r < end) {  // uniform: skip batches past this wave's slots
        const int s = base + 64 * r + lane;
        const int e = ev[r];
        const bool v = e >= 0 && e < E;
        const uint64_t peers = peers_of(e, v, nbits);
        const int rank = __popcll(peers & below);
        int prior = 0;
        if (v) prior = cnt[wave][e];
        if (v) bucket[s_off[e] + prior + rank] = s;
        if (v && rank == 0) cnt[wave][e] = prior + __popcll(peers);
      }
    }
  }
  if (tid <= kXcds) counters[tid] = 0u;
}

// One workgroup per (token, 1024-column chunk); each thread one float4 of
// the output row (M % 4 == 0) or one float.  The slot weights of the token
// are uniform over the workgroup.
template <bool VEC>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ ys,
                                                          const float* __restrict__ p,
                                                          const int32_t* __restrict__ ids, int E,
                                                          float* __restrict__ y, int top_k, int M, int t0) {
  const int t = t0 + static_cast<int>(blockIdx.y);
  const int c = (blockIdx.x * 256 + threadIdx.x) * (VEC ? 4 : 1);
  if (c >= M) return;
  const size_t slot0 = static_cast<size_t>(t) * top_k;
  if constexpr (VEC) {
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int k = 0; k < top_k; ++k) {
      const int e = ids[slot0 + k];
      if (e < 0 || e >= E) continue;
      const float w = p[slot0 + k];
      const float4 v = *reinterpret_cast<const float4*>(ys + (slot0 + k) * M + c);
      acc.x = __builtin_fmaf(w, v.x, acc.x);
      acc.y = __builtin_fmaf(w, v.y, acc.y);
      acc.z = __builtin_fmaf(w, v.z, acc.z);
      acc.w = __builtin_fmaf(w, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + static_cast<size_t>(t) * M + c) = acc;
  } else {
    float acc = 0.0f;
    for (int k = 0; k < top_k; ++k) {
      const int e = ids[slot0 + k];
      if (e >= 0 && e < E) acc = __builtin_fmaf(p[slot0 + k], ys[(slot0 + k) * M + c], acc);
    }
    y[static_cast<size_t>(t) * M + c] = acc;
  }
}

}  // namespace qmm

using namespace qmm;

// One grouped call; with `routed`, the route tables already in ws (left by
// an earlier grouped call on ws with the same ids, T, top_k and E) are used
// instead of being prepared again.
// Ordered weighted combine of the per-slot rows in scratch into y[T][M].
static int combine(const float* scratch, const float* expert_weights, const int32_t* ids, int64_t E, float* y,
                   int64_t T, int64_t top_k, int64_t M, hipStream_t st) {
  const bool vec = (M % 4) == 0;
  const int per_block = vec ? 1024 : 256;
  constexpr int64_t kMaxGridY = 65535;
  for (int64_t t0 = 0; t0 < T; t0 += kMaxGridY) {
    const dim3 grid(static_cast<unsigned>((M + per_block - 1) / per_block),
                    static_cast<unsigned>(std::min(kMaxGridY, T - t0)));
    if (vec)
      hipLaunchKernelGGL(moe_combine_kernel<true>, grid, dim3(256), 0, st, scratch, expert_weights, ids,
                         static_cast<int>(E), y, static_cast<int>(top_k), static_cast<int>(M), static_cast<int>(t0));
    else
      hipLaunchKernelGGL(moe_combine_kernel<false>, grid, dim3(256), 0, st, scratch, expert_weights, ids,
                         static_cast<int>(E), y, static_cast<int>(top_k), static_cast<int>(M), static_cast<int>(t0));
    const int rc = launch_status();
    if (rc != QMM_OK) return rc;
  }
  return QMM_OK;
}

// hq != nullptr: the fused SwiGLU call (Q8_1 rows into hq instead of fp32
// rows into y; no routing weights).
static int grouped_call(bool routed, int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                        int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token, const int32_t* ids,
                        const float* expert_weights, int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes,
                        void* stream, void* hq = nullptr) {
  if (fmt != QMM_Q4_K && fmt != QMM_Q5_K && fmt != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  if (hq != nullptr) {
    // gate and up halves of 128-row multiples, on the whole-K Q4_K / Q5_K tiles
    if (fmt == QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
    if (M < 256 || (M % 256) != 0) return QMM_ERR_SHAPE;
  }
  if (E < 1 || E > kMoeMaxE || M < 1 || M > (1 << 30) || K < kQK || (K % kQK) != 0 || K / kQK > (1 << 16) ||
      T < 1 || top_k < 1 || top_k > E || top_k > kMoeMaxTopK || T * top_k > (1 << 30))
    return QMM_ERR_SHAPE;
  // work entries (m_tile, column tile) are numbered in 32-bit
  if (((M + kMoeBM - 1) / kMoeBM) * moe_max_ctiles(T * top_k, E) > (int64_t{1} << 30)) return QMM_ERR_SHAPE;
  if (x_rows_per_token != 1 && x_rows_per_token != top_k) return QMM_ERR_SHAPE;
  const int64_t row_bytes = (K / kQK) * (fmt == QMM_Q4_K ? kQ4Bytes : fmt == QMM_Q5_K ? kQ5Bytes : kQ6Bytes);
  // Q4_K / Q5_K blocks are read with 16-byte loads, Q6_K blocks with 2-byte aligned ones
  const int64_t stride_align = fmt == QMM_Q6_K ? 2 : 16;
  if (expert_stride_bytes < M * row_bytes || (expert_stride_bytes % stride_align) != 0) return QMM_ERR_SHAPE;
  if (!w || !xq || !ids || (!y && !hq) || !ws) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(ids) || (y && !aligned16(y)) || (hq && !aligned16(hq)) ||
      !aligned16(ws) ||
      (expert_weights && !aligned16(expert_weights)))
    return QMM_ERR_ALIGN;
  const MoeLayout L = moe_layout(ws, M, K, T, E, top_k, expert_weights != nullptr);
  if (ws_bytes < L.bytes) return QMM_ERR_WORKSPACE;
  hipStream_t st = to_stream(stream);
  const int n = static_cast<int>(T * top_k);
  int rc;
  if (!routed) {
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, ids, n, static_cast<int>(E),
                       L.counts, L.offsets, L.ct_off, L.bucket, L.counters);
    rc = launch_status();
    if (rc != QMM_OK) return rc;
  }
  float* out = expert_weights ? L.scratch : y;
  rc = mmq_moe_launch(fmt, static_cast<const uint8_t*>(w), expert_stride_bytes, static_cast<int>(M),
                      static_cast<int>(K / kQK), static_cast<const uint8_t*>(xq), out, static_cast<uint8_t*>(hq),
                      L.counters,
                      L.counts, L.offsets, L.bucket, L.ct_off, L.chunks,
                      static_cast<int>(moe_max_ctiles(T * top_k, E)), static_cast<int>(E),
                      static_cast<int>(top_k), static_cast<int>(x_rows_per_token), st);
  if (rc != QMM_OK || !expert_weights) return rc;
  return combine(L.scratch, expert_weights, ids, E, y, T, top_k, M, st);
}

extern "C" int moe_grouped_mmq(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                               int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                               const int32_t* ids, const float* expert_weights, int64_t T,
                               int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream) {
  return grouped_call(false, fmt, w, E, M, K, expert_stride_bytes, xq, x_rows_per_token, ids, expert_weights,
                           T, top_k, y, ws, ws_bytes, stream);
}

extern "C" int moe_grouped_mmq_swiglu(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                                      int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                                      const int32_t* ids, int64_t T, int64_t top_k, void* hq, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!hq) return QMM_ERR_NULL;
  return grouped_call(false, fmt, w, E, M, K, expert_stride_bytes, xq, x_rows_per_token, ids, nullptr, T, top_k,
                      nullptr, ws, ws_bytes, stream, hq);
}

extern "C" int moe_grouped_mmq_routed(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                                      int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                                      const int32_t* ids, const float* expert_weights, int64_t T,
                                      int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream) {
  return grouped_call(true, fmt, w, E, M, K, expert_stride_bytes, xq, x_rows_per_token, ids, expert_weights,
                           T, top_k, y, ws, ws_bytes, stream);
}

// The routed FFN layer in one call: route preparation, the gate||up product
// with SwiGLU -> Q8_1 in its epilogue writing the down product's activation
// chunks directly (no Q8_1 rows, no second repack), the weighted down product
// and the ordered combine.
extern "C" int moe_ffn(int fmt_gu, const void* w_gu, int64_t stride_gu, int fmt_dn, const void* w_dn,
                       int64_t stride_dn, int64_t E, int64_t H, int64_t F, const void* xq, const int32_t* ids,
                       const float* expert_weights, int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes,
                       void* stream) {
  if (fmt_gu != QMM_Q4_K && fmt_gu != QMM_Q5_K) return QMM_ERR_UNSUPPORTED;
  if (fmt_dn != QMM_Q4_K && fmt_dn != QMM_Q5_K && fmt_dn != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  if (E < 1 || E > kMoeMaxE || H < kQK || (H % kQK) != 0 || H / kQK > (1 << 16) || F < kQK || (F % kQK) != 0 ||
      2 * F > (1 << 30) || H > (1 << 30) || T < 1 || top_k < 1 || top_k > E || top_k > kMoeMaxTopK ||
      T * top_k > (1 << 30))
    return QMM_ERR_SHAPE;
  const int64_t maxw = std::max(2 * F, H);
  if (((maxw + kMoeBM - 1) / kMoeBM) * moe_max_ctiles(T * top_k, E) > (int64_t{1} << 30)) return QMM_ERR_SHAPE;
  const auto rowb = [](int fmt, int64_t K) {
    return (K / kQK) * (fmt == QMM_Q4_K ? kQ4Bytes : fmt == QMM_Q5_K ? kQ5Bytes : kQ6Bytes);
  };
  if (stride_gu < 2 * F * rowb(fmt_gu, H) || (stride_gu % 16) != 0) return QMM_ERR_SHAPE;
  if (stride_dn < H * rowb(fmt_dn, F) || (stride_dn % (fmt_dn == QMM_Q6_K ? 2 : 16)) != 0) return QMM_ERR_SHAPE;
  if (!w_gu || !w_dn || !xq || !ids || !expert_weights || !y || !ws) return QMM_ERR_NULL;
  if (!aligned16(w_gu) || !aligned16(w_dn) || !aligned16(xq) || !aligned16(ids) || !aligned16(expert_weights) ||
      !aligned16(y) || !aligned16(ws))
    return QMM_ERR_ALIGN;
  const FfnLayout L = ffn_layout(ws, H, F, T, E, top_k);
  if (ws_bytes < L.bytes) return QMM_ERR_WORKSPACE;
  hipStream_t st = to_stream(stream);
  const int n = static_cast<int>(T * top_k);
  const MoeLayout& D = L.dn;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, ids, n, static_cast<int>(E), D.counts,
                     D.offsets, D.ct_off, D.bucket, D.counters);
  int rc = launch_status();
  if (rc != QMM_OK) return rc;
  const int mct = static_cast<int>(moe_max_ctiles(T * top_k, E));
  // gate||up: its own repack into chunks_gu (zeroing both queues), the
  // SwiGLU epilogue writing the down chunks into D.chunks
  rc = mmq_moe_launch(fmt_gu, static_cast<const uint8_t*>(w_gu), stride_gu, static_cast<int>(2 * F),
                      static_cast<int>(H / kQK), static_cast<const uint8_t*>(xq), nullptr, D.chunks, D.counters,
                      D.counts, D.offsets, D.bucket, D.ct_off, L.chunks_gu, mct, static_cast<int>(E),
                      static_cast<int>(top_k), 1, st, D.chunks, static_cast<int>(F / kQK), true);
  if (rc != QMM_OK) return rc;
  // down on those chunks (no repack), per-slot rows into the scratch
  rc = mmq_moe_launch(fmt_dn, static_cast<const uint8_t*>(w_dn), stride_dn, static_cast<int>(H),
                      static_cast<int>(F / kQK), nullptr, D.scratch, nullptr, D.counters, D.counts, D.offsets,
                      D.bucket, D.ct_off, D.chunks, mct, static_cast<int>(E), static_cast<int>(top_k), top_k, st,
                      nullptr, 0, false);
  if (rc != QMM_OK) return rc;
  return combine(D.scratch, expert_weights, ids, E, y, T, top_k, H, st);
}
