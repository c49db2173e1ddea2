// Internal helpers shared by the libqmm translation units (device and host).
//
// Pages cited (title, then section):
//   [8e]  minfer ch. 06, "06 · 8e/8e② — decode MMVQ: dp4a integer dot products
//         + the llama.cpp launch table"
//   [MMQ] ZINC, "ZINC MMQ v2 — Fused Q4_K×Q8_1 Tensor-Core GEMM (beat llama.cpp)"
//   [GAP] ZINC, "Prefill Gap Closure Plan — ZINC CUDA vs llama.cpp"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "qmm.h"

namespace qmm {

constexpr int kQK = 256;       // weights per K-quant super-block
constexpr int kQB = 32;        // activations per Q8_1 block
constexpr int kQ4Bytes = 144;  // Q4_K super-block bytes
constexpr int kQ5Bytes = 176;  // Q5_K super-block bytes
constexpr int kQ6Bytes = 210;  // Q6_K super-block bytes
constexpr int kQ8Bytes = 40;   // Q8_1 block bytes
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int kMoeMaxE = 512;  // experts per grouped MoE call

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t to_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Map the runtime's last error (after an enqueue) to a status.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? QMM_OK : QMM_ERR_HIP;
}

// Compute units of the current device, cached per device id.
int device_cu_count();

// ----------------------------------------------------------------------------
// Device side
// ----------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 16-byte load from a 4-byte aligned address (one dwordx4 load).
struct __attribute__((aligned(4))) u32x4_a4 { uint32_t v[4]; };

__device__ __forceinline__ uint4 ld16_a4(const void* p) {
  const u32x4_a4 t = *reinterpret_cast<const u32x4_a4*>(p);
  return make_uint4(t.v[0], t.v[1], t.v[2], t.v[3]);
}

__device__ __forceinline__ uint4 ld16_a16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte aligned load marked non-temporal (streamed once; keeps L2 for data
// that is reused).
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes from a 2-byte aligned address: aligned dword loads joined with a
// byte funnel shift.  Q6_K blocks are 210 bytes, so every other block starts
// at 2 mod 4.  The fifth dword is read only when the address is misaligned,
// so nothing past p + 16 is touched for aligned addresses.
// The aligned base is formed by pointer arithmetic on p (not through an
// integer), so the loads keep p's global address space instead of becoming
// flat loads (which also count against the LDS wait counter).
__device__ __forceinline__ uint4 ld16_a2(const uint8_t* p) {
  const uint32_t sh = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) & 3u);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p - sh);
  const uint32_t w0 = base[0], w1 = base[1], w2 = base[2], w3 = base[3];
  const uint32_t w4 = sh ? base[4] : 0u;
  return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh),
                    __builtin_amdgcn_alignbyte(w3, w2, sh), __builtin_amdgcn_alignbyte(w4, w3, sh));
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// IEEE binary16 bits <-> float (exact widening; round-to-nearest-even narrowing).
__device__ __forceinline__ float h2f(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}
__device__ __forceinline__ uint32_t f2h_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Four int8 x int8 products summed into c ([8e] §2: the 4-way integer dot).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// The same with c = 0, as one instruction: the compiler's accumulating form
// would first zero a register for it.
__device__ __forceinline__ int dot4_0(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// An int32 sum started at the bits of 1.5 * 2^23 and read as fp32 is exactly
// 1.5 * 2^23 + sum while |sum| < 2^22; a product a * sum then takes one fma
// against the constant -a * 1.5 * 2^23 (exact whenever a has at most 22
// significant bits), with no int-to-float conversion.
constexpr uint32_t kMagicBits = 0x4B400000u;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// dot4 with c = the bits of 1.5 * 2^23 (held in a scalar register), as one
// instruction.
__device__ __forceinline__ int dot4_magic(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(kMagicBits));
  return r;
}

// Q4_K packed 6-bit scale and min of sub-block j (0..7).  s0, s1, s2 are the
// 12 packed bytes as little-endian dwords (bytes 0-3, 4-7, 8-11).  Packing as
// read for the Q4_K format (GGUF K-quant layout):
//   j < 4:  sc = S[j] & 63,                 m = S[j+4] & 63
//   j >= 4: sc = S[j+4] & 15 | (S[j-4]>>6)<<4, m = S[j+4]>>4 | (S[j]>>6)<<4
__device__ __forceinline__ void q4k_scale_min(int j, uint32_t s0, uint32_t s1, uint32_t s2,
                                              int& sc, int& m) {
  const int k = (j & 3) * 8;
  const int sc_lo = (s0 >> k) & 63, m_lo = (s1 >> k) & 63;
  const int sc_hi = ((s2 >> k) & 15) | (((s0 >> (k + 6)) & 3) << 4);
  const int m_hi = ((s2 >> (k + 4)) & 15) | (((s1 >> (k + 6)) & 3) << 4);
  sc = j < 4 ? sc_lo : sc_hi;
  m = j < 4 ? m_lo : m_hi;
}

// LDS byte address of a (generic) pointer into shared memory: a flat
// address in the LDS aperture carries the LDS offset in its low 32 bits.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane
// (global_load_lds_dwordx4; the LDS base goes through M0).  Written as
// inline assembly so the compiler does not track it: its own tracking treats
// every later LDS read as a possible alias and waits for all loads in flight,
// which would serialise a prefetch into the work that precedes its use.  The
// caller waits for these copies explicitly (wait_vmcnt, plus a barrier when
// other waves read the data).  M0 is a reserved register the compiler may
// hold a value in, so the sequence saves and restores it (the load takes its
// LDS base from M0 when it is issued).  NT marks the load non-temporal (data
// read once, kept out of the way of reused lines).
template <bool NT = false>
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  if constexpr (NT) {
    __asm__ volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(src), "s"(m0v)
                     : "memory");
  } else {
    __asm__ volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(src), "s"(m0v)
                     : "memory");
  }
}

// 4 bytes per lane from global memory into LDS at lds + 4 * lane
// (global_load_lds_dword), the same way as dma16: lanes may gather from any
// addresses, so one instruction can rearrange 256 bytes into LDS order.
__device__ __forceinline__ void dma4(const uint8_t* src, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  __asm__ volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\t"
                   "s_mov_b32 m0, %0"
                   : "=&s"(saved)
                   : "v"(src), "s"(m0v)
                   : "memory");
}

// Wait until at most N of this wave's vector memory operations (loads,
// stores, the copies above) are outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Q6_K signed values q6 - 32 = low nibble + 16 * (hi - 2): a byte-table lookup
// (v_perm) maps the two high bits hi to the int8 16 * (hi - 2), whose low
// nibble is zero, so OR-ing in the low nibble gives the value.
constexpr uint32_t kQ6HiTable = 0x1000F0E0u;  // bytes -32, -16, 0, 16 as int8

// Wave64 reductions.
// Sum over the 64 lanes (all active), returned in every lane: inclusive
// prefix sums inside each 16-lane row by DPP row shifts (lanes shifted in
// from outside the row read 0), so lane 15 of each row holds the row's sum;
// the four row sums are then read out and added in row order.  No LDS
// traffic (a butterfly of lane shuffles takes six LDS-crossbar round trips).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true);
  return v + __builtin_bit_cast(float, s);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0x111>(v);  // row_shr:1
  v = dpp_add<0x112>(v);  // row_shr:2
  v = dpp_add<0x114>(v);  // row_shr:4
  v = dpp_add<0x118>(v);  // row_shr:8
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 63));
  return (r0 + r1) + (r2 + r3);
}

// A value from another lane of the same group of eight, by DPP (no LDS
// crossbar): CTRL 0xb1 and 0x4e are the quad permutations lane ^ 1 and
// lane ^ 2, 0x141 mirrors each half-row (lane i of an 8-lane group takes lane
// 7 - i, in the other quad).  Used where the group's values are all equal
// within each quad, so the mirror acts as lane ^ 4.
template <int CTRL>
__device__ __forceinline__ float lane8_xchg(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int lane8_xchg(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}

// Quantize one 32-activation block to Q8_1 with eight consecutive lanes.
// Lane `part` (0..7) holds x[4*part .. 4*part+3]; all eight lanes must be
// active (they exchange values).  Steps of [8e] §3.2 (max |x|, d = am/127,
// reciprocal, round to nearest even, clamp, pack, sum), in IEEE fp32 with
// no contraction so the bytes are reproducible; a subnormal d is taken as 0.  Returns this lane's four
// int8 values packed little-endian, the fp32 scale d (stored as f16) and
// the block's integer sum (in every lane of the group).  Every step is
// independent of the order of the lanes, so any caller gets the same bytes.
__device__ __forceinline__ void q8_1_block_8lanes_vals(float4 v, uint32_t& packed, float& d, int& s) {
#pragma clang fp contract(off)
  float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  am = fmaxf(am, lane8_xchg<0xb1>(am));   // quad_perm [1, 0, 3, 2]: lane ^ 1
  am = fmaxf(am, lane8_xchg<0x4e>(am));   // quad_perm [2, 3, 0, 1]: lane ^ 2
  am = fmaxf(am, lane8_xchg<0x141>(am));  // row_half_mirror: the other quad of the 8
  d = am / 127.0f;
  // a subnormal scale counts as zero (its reciprocal may overflow and its
  // f16 rounding is 0): the block is stored as zeros
  const float di = d >= 0x1p-126f ? 1.0f / d : 0.0f;
  const int q0 = max(-128, min(127, static_cast<int>(rintf(v.x * di))));
  const int q1 = max(-128, min(127, static_cast<int>(rintf(v.y * di))));
  const int q2 = max(-128, min(127, static_cast<int>(rintf(v.z * di))));
  const int q3 = max(-128, min(127, static_cast<int>(rintf(v.w * di))));
  packed = (static_cast<uint32_t>(q0) & 255u) | ((static_cast<uint32_t>(q1) & 255u) << 8) |
           ((static_cast<uint32_t>(q2) & 255u) << 16) | (static_cast<uint32_t>(q3) << 24);
  s = q0 + q1 + q2 + q3;
  s += lane8_xchg<0xb1>(s);
  s += lane8_xchg<0x4e>(s);
  s += lane8_xchg<0x141>(s);
}

// The same, stored as the block's 40 bytes at dst (4-byte aligned; nothing
// is stored when `store` is false).
__device__ __forceinline__ void q8_1_block_8lanes(float4 v, int part, uint8_t* dst, bool store) {
  uint32_t packed;
  float d;
  int s;
  q8_1_block_8lanes_vals(v, packed, d, s);
  if (!store) return;
  reinterpret_cast<uint32_t*>(dst + 4)[part] = packed;
  if (part == 0) {
    reinterpret_cast<uint32_t*>(dst)[0] = f2h_bits(d);  // f16 d, zero pad
    reinterpret_cast<int32_t*>(dst + 36)[0] = s;
  }
}

// One 32-activation block quantized by two lanes, lane and lane ^ 32, each
// holding 16 of its values (any split): the same steps as
// q8_1_block_8lanes_vals, so the same bytes.  Both lanes must be active.
// Returns this lane's 16 int8 values packed four per dword (h[4k .. 4k+3]
// in dword k, little-endian), the fp32 scale d and the block's integer sum
// (in both lanes).
__device__ __forceinline__ void q8_1_block_2lanes_vals(const float (&h)[16], uint32_t (&packed)[4], float& d,
                                                       int& s) {
#pragma clang fp contract(off)
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(h[i]));
  am = fmaxf(am, __shfl_xor(am, 32));
  d = am / 127.0f;
  const float di = d >= 0x1p-126f ? 1.0f / d : 0.0f;
  s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t p = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = max(-128, min(127, static_cast<int>(rintf(h[4 * k + j] * di))));
      s += q;
      p |= (static_cast<uint32_t>(q) & 255u) << (8 * j);
    }
    packed[k] = p;
  }
  s += __shfl_xor(s, 32);
}

// SwiGLU of one gate value g and its up value u: silu(g) * u.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace qmm
