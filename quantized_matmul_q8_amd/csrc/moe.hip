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
// for 64 slots at a time, lanes with the same expert find each other with one
// ballot per id bit, so a lane's rank among equal ids is a popcount.  Pass 1
// counts per (wave, expert), a scan turns counts into offsets, pass 2 repeats
// the ranking and writes every slot to its place.  It also writes the work
// prefix (m_tiles * ceil(count / 32) per expert) and zeroes the queue
// counters that the grouped kernel claims tiles from.
//
// The combine y[t] = sum_k p[t][k] * y_slot[t*top_k + k] runs in increasing
// k with no atomics, so results are bit-reproducible.
#include "qmm_common.hpp"

namespace qmm {

constexpr int kMoeMaxE = 512;
constexpr int kMoeMaxTopK = 64;
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr size_t kMoeCounterBytes = 256;
constexpr int kMoeBN = 32;   // routed tokens per tile (must match the grouped kernel)
constexpr int kMoeBM = 128;  // weight rows per tile

int mmq_moe_launch(int fmt, const uint8_t* w, int64_t stride, int M, int nb, const uint8_t* xq,
                   float* out, unsigned* counters, const int32_t* counts, const int32_t* offsets,
                   const int32_t* bucket, const int32_t* work_off, int E, int top_k,
                   int rows_per_token, hipStream_t st);

struct MoeLayout {
  unsigned* counters;
  int32_t* counts;
  int32_t* offsets;
  int32_t* work_off;
  int32_t* bucket;
  float* scratch;
  size_t bytes;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static MoeLayout moe_layout(void* ws, int64_t M, int64_t T, int64_t E, int64_t top_k) {
  MoeLayout L{};
  uint8_t* b = static_cast<uint8_t*>(ws);
  size_t off = kMoeCounterBytes;
  const size_t ints = static_cast<size_t>(E) + 2 * static_cast<size_t>(E + 1) + static_cast<size_t>(T * top_k);
  L.counters = reinterpret_cast<unsigned*>(b);
  L.counts = reinterpret_cast<int32_t*>(b + off);
  L.offsets = L.counts + E;
  L.work_off = L.offsets + (E + 1);
  L.bucket = L.work_off + (E + 1);
  off = align_up(off + ints * 4, 256);
  L.scratch = reinterpret_cast<float*>(b + off);
  off += static_cast<size_t>(T * top_k) * static_cast<size_t>(M) * 4;
  L.bytes = off;
  return L;
}

size_t moe_workspace_bytes(int64_t M, int64_t T, int64_t E, int64_t top_k) {
  return moe_layout(nullptr, M, T, E, top_k).bytes;
}

__device__ __forceinline__ uint64_t peers_of(int e, bool v, int nbits) {
  uint64_t peers = __ballot(v);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(v && bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const int32_t* __restrict__ ids, int n, int E, int mt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ work_off, int32_t* __restrict__ bucket,
    unsigned* __restrict__ counters) {
  __shared__ int cnt[kRouteWaves][kMoeMaxE];
  __shared__ int s_off[kMoeMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kRouteWaves * kMoeMaxE; i += kRouteThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int per = (n + kRouteWaves - 1) / kRouteWaves;
  const int beg = wave * per, end = min(n, beg + per);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // pass 1: per-(wave, expert) counts
  for (int base = beg; base < end; base += 64) {
    const int s = base + lane;
    const int e = s < end ? ids[s] : -1;
    const bool v = e >= 0 && e < E;
    const uint64_t peers = peers_of(e, v, nbits);
    if (v && __popcll(peers & below) == 0) cnt[wave][e] += __popcll(peers);
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
    s_off[e] = run;  // total, turned into the offset below
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, woff = 0;
    for (int e = 0; e < E; ++e) {
      const int c = s_off[e];
      s_off[e] = off;
      offsets[e] = off;
      work_off[e] = woff;
      off += c;
      woff += ((c + kMoeBN - 1) / kMoeBN) * mt;
    }
    offsets[E] = off;
    work_off[E] = woff;
  }
  __syncthreads();
  // pass 2: stable scatter of slot ids
  for (int base = beg; base < end; base += 64) {
    const int s = base + lane;
    const int e = s < end ? ids[s] : -1;
    const bool v = e >= 0 && e < E;
    const uint64_t peers = peers_of(e, v, nbits);
    const int rank = __popcll(peers & below);
    int prior = 0;
    if (v) prior = cnt[wave][e];
    if (v) bucket[s_off[e] + prior + rank] = s;
    if (v && rank == 0) cnt[wave][e] = prior + __popcll(peers);
  }
  if (tid <= kXcds) counters[tid] = 0u;
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ ys,
                                                          const float* __restrict__ p,
                                                          const int32_t* __restrict__ ids, int E,
                                                          float* __restrict__ y, int T, int top_k,
                                                          int M) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * M) return;
  const int t = static_cast<int>(i / M), c = static_cast<int>(i % M);
  float acc = 0.0f;
  for (int k = 0; k < top_k; ++k) {
    const int s = t * top_k + k;
    const int e = ids[s];
    if (e >= 0 && e < E) acc = __builtin_fmaf(p[s], ys[static_cast<int64_t>(s) * M + c], acc);
  }
  y[i] = acc;
}

}  // namespace qmm

using namespace qmm;

extern "C" int moe_grouped_mmq(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                               int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                               const int32_t* ids, const float* expert_weights, int64_t T,
                               int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (fmt != QMM_Q4_K && fmt != QMM_Q6_K) return QMM_ERR_UNSUPPORTED;
  if (E < 1 || E > kMoeMaxE || M < 1 || M > (1 << 30) || K < kQK || (K % kQK) != 0 || T < 1 ||
      top_k < 1 || top_k > E || top_k > kMoeMaxTopK || T * top_k > (1 << 30))
    return QMM_ERR_SHAPE;
  if (x_rows_per_token != 1 && x_rows_per_token != top_k) return QMM_ERR_SHAPE;
  const int64_t row_bytes = (K / kQK) * (fmt == QMM_Q4_K ? kQ4Bytes : kQ6Bytes);
  // Q4_K blocks are read with 16-byte loads, Q6_K blocks with 2-byte aligned ones
  const int64_t stride_align = fmt == QMM_Q4_K ? 16 : 2;
  if (expert_stride_bytes < M * row_bytes || (expert_stride_bytes % stride_align) != 0) return QMM_ERR_SHAPE;
  if (!w || !xq || !ids || !y || !ws) return QMM_ERR_NULL;
  if (!aligned16(w) || !aligned16(xq) || !aligned16(ids) || !aligned16(y) || !aligned16(ws) ||
      (expert_weights && !aligned16(expert_weights)))
    return QMM_ERR_ALIGN;
  const MoeLayout L = moe_layout(ws, M, T, E, top_k);
  if (ws_bytes < L.bytes) return QMM_ERR_WORKSPACE;
  hipStream_t st = to_stream(stream);
  const int n = static_cast<int>(T * top_k);
  const int mt = static_cast<int>((M + kMoeBM - 1) / kMoeBM);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, st, ids, n, static_cast<int>(E),
                     mt, L.counts, L.offsets, L.work_off, L.bucket, L.counters);
  int rc = launch_status();
  if (rc != QMM_OK) return rc;
  float* out = expert_weights ? L.scratch : y;
  rc = mmq_moe_launch(fmt, static_cast<const uint8_t*>(w), expert_stride_bytes, static_cast<int>(M),
                      static_cast<int>(K / kQK), static_cast<const uint8_t*>(xq), out, L.counters,
                      L.counts, L.offsets, L.bucket, L.work_off, static_cast<int>(E),
                      static_cast<int>(top_k), static_cast<int>(x_rows_per_token), st);
  if (rc != QMM_OK || !expert_weights) return rc;
  const int64_t total = T * M;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st,
                     L.scratch, expert_weights, ids, static_cast<int>(E), y, static_cast<int>(T),
                     static_cast<int>(top_k), static_cast<int>(M));
  return launch_status();
}
