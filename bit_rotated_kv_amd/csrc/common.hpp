// Shared device/host helpers of the OSCAR gfx950 kernels: layout arithmetic, bf16/fp16 bit
// conversions, matrix-core operand types and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kPage = 16;       // tokens per page
constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kMetaBytes = 128; // 16 token slots x {sK, zK, sV, zV} bf16

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ layout sizes
__host__ __device__ inline int64_t qpage_head_bytes(int d, int bits) { return 4LL * d * bits + kMetaBytes; }
__host__ __device__ inline int64_t bf16_page_head_bytes(int d) { return 64LL * d; }
__host__ __device__ inline int lane_chunk_bytes(int d, int bits) { return d * bits / 32; }  // K part; V part same

// Byte address of page-head (page, kv) in the pool arena. Pages below off4 are INT2 pages,
// pages at or above it INT4 pages stacked after the INT2 region.
__device__ inline const uint8_t* page_head_addr(const uint8_t* pool, int64_t page, int kv, int hkv, int d,
                                                int64_t off4) {
  const int64_t p2 = qpage_head_bytes(d, 2) * hkv;
  if (page < off4) return pool + page * p2 + (int64_t)kv * qpage_head_bytes(d, 2);
  const int64_t p4 = qpage_head_bytes(d, 4) * hkv;
  return pool + off4 * p2 + (page - off4) * p4 + (int64_t)kv * qpage_head_bytes(d, 4);
}

// Pointer into global memory (address space 1): loads through it are global loads, also where
// the address was assembled from scalar registers.
template <typename T>
using GPtr = const __attribute__((address_space(1))) T*;

// ------------------------------------------------------------------ number formats
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// ------------------------------------------------------------------ wavefront reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP row shift right by N lanes inside each 16-lane row: lane l reads lane l-N (lanes whose
// source falls outside the row read 0).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_shr(uint32_t v) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, false);
}
// DPP row shift left: lane l reads lane l+N of its row (0 outside the row).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_shl(uint32_t v) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, false);
}
// DPP move with a bank mask: lanes of the 4-lane banks set in BANKS receive src from the lane
// that CTRL selects; the other lanes keep old. Selecting by bank mask keeps the move
// unconditional: a data-dependent select around a DPP move may be turned into a branch, and a
// DPP move executed under a narrowed exec mask reads inactive source lanes as invalid.
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANKS, false);
}
template <int N, int BANKS>
__device__ __forceinline__ uint32_t dpp_row_shr_into(uint32_t old, uint32_t src) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return dpp_into<0x110 + N, BANKS>(old, src);
}
template <int N, int BANKS>
__device__ __forceinline__ uint32_t dpp_row_shl_into(uint32_t old, uint32_t src) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return dpp_into<0x100 + N, BANKS>(old, src);
}
template <int N, int BANKS>
__device__ __forceinline__ float dpp_row_shr_into(float old, float src) {
  return __uint_as_float(dpp_row_shr_into<N, BANKS>(__float_as_uint(old), __float_as_uint(src)));
}
// DPP row rotate right by N lanes inside each 16-lane row.
template <int N>
__device__ __forceinline__ float dpp_row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF,
                                                               false));
}
// Wave-uniform copy of a value (the compiler treats the result as scalar).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------------ exact group quantiser
// Quantiser decision in fp32, operation by operation with multiply-add contraction switched off
// (c*max - c*min must not become one fused operation): lo = c*min, hi = c*max,
// s = bf16(fp32(hi - lo)/L), z = bf16(lo), code = clamp(rint_even(fp32(clamp(x,lo,hi) - z)/s), 0, L).
struct QuantGrid {
  float lo, hi, s, z;
  float rs;                 // hardware reciprocal of s (estimate for quant_code)
  uint32_t s_bits, z_bits;
};

__device__ __forceinline__ QuantGrid make_grid(float mn, float mx, float clip, int levels) {
#pragma clang fp contract(off)
  QuantGrid g;
  g.lo = clip * mn;
  g.hi = clip * mx;
  const float s32 = __fdiv_rn(g.hi - g.lo, (float)levels);
  g.s_bits = f32_to_bf16_bits(s32);
  g.z_bits = f32_to_bf16_bits(g.lo);
  g.s = bf16_bits_to_f32(g.s_bits);
  g.z = bf16_bits_to_f32(g.z_bits);
  g.rs = __builtin_amdgcn_rcpf(g.s);
  return g;
}

// The quotient t = fl(d / s) only feeds rint, so it is first estimated as d * rcp(s): the hardware
// reciprocal is within 1 ulp, the estimate within 2^-17 of d / s for |t| < 32, and the correctly
// rounded quotient within 2^-19. Unless the estimate lies within 2^-14 of a rounding midpoint
// k + 1/2 (or is not below 32 in magnitude, or not a number), both round to the same integer.
// quant_code_fast returns the code of the estimate and sets `redo` in those cases, where
// quant_code_exact (the correctly rounded division) decides; quant_code chains the two. Every
// variant returns the code of the exact rule.
// (branch-free: the clamps are median-of-three, the tests combine with bitwise operators)
__device__ __forceinline__ uint32_t quant_code_fast(float x, const QuantGrid& g, int levels, bool& redo) {
#pragma clang fp contract(off)
  const float xc = __builtin_amdgcn_fmed3f(x, g.lo, g.hi);
  const float t = (xc - g.z) * g.rs;
  redo = (g.s != 0.0f) & (!(fabsf(t) < 32.0f) | (fabsf(__builtin_amdgcn_fractf(t) - 0.5f) <= 0x1p-14f));
  const float r = __builtin_amdgcn_fmed3f(rintf(t), 0.0f, (float)levels);
  return g.s == 0.0f ? 0u : (uint32_t)r;
}

__device__ __forceinline__ uint32_t quant_code_exact(float x, const QuantGrid& g, int levels) {
#pragma clang fp contract(off)
  if (g.s == 0.0f) return 0u;
  const float xc = fminf(fmaxf(x, g.lo), g.hi);
  const float t = __fdiv_rn(xc - g.z, g.s);
  return (uint32_t)fminf(fmaxf(rintf(t), 0.0f), (float)levels);
}

__device__ __forceinline__ uint32_t quant_code(float x, const QuantGrid& g, int levels) {
  bool redo;
  const uint32_t c = quant_code_fast(x, g, levels, redo);
  return redo ? quant_code_exact(x, g, levels) : c;
}

// ------------------------------------------------------------------ history code placement
// Word index (within the lane chunk) and bit position of a key / value code, for page slot t and
// channel ch (the layouts documented in oscar.h).
struct CodePos {
  int lane, word, bit;
};

__host__ __device__ inline CodePos key_pos(int bits, int t, int ch) {
  const int kk = ch / 32, g = (ch % 32) / 8, m = (ch % 8) / 2, hf = ch % 2;
  CodePos p;
  p.lane = 16 * g + t;
  if (bits == 2) {
    p.word = kk / 2;
    p.bit = 8 * (kk % 2) + 2 * m + 16 * hf;
  } else {
    p.word = kk;
    p.bit = 4 * m + 16 * hf;
  }
  return p;
}

__host__ __device__ inline CodePos value_pos(int bits, int t, int ch) {
  const int nb = ch / 16, c = ch % 16, g = t / 4, m = (t % 4) / 2, hf = t % 2;
  CodePos p;
  p.lane = 16 * g + c;
  if (bits == 2) {
    p.word = nb / 4;
    p.bit = 2 * (nb % 4) + 8 * m + 16 * hf;
  } else {
    p.word = nb / 2;
    p.bit = 4 * (nb % 2) + 8 * m + 16 * hf;
  }
  return p;
}

// BF16 page-head element offsets (in bf16 units).
__host__ __device__ inline int bf16_key_index(int d, int t, int ch) {
  const int kk = ch / 32, g = (ch % 32) / 8, i = ch % 8;
  return ((g * 16 + t) * (d / 32) + kk) * 8 + i;
}
__host__ __device__ inline int bf16_value_index(int d, int t, int ch) {
  const int nb = ch / 16, c = ch % 16, g = t / 4, r = t % 4;
  return 16 * d + ((g * 16 + c) * (d / 16) + nb) * 4 + r;
}

}  // namespace oscar
